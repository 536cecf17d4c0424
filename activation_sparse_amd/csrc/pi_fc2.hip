// pi_fc2.hip - FC2 as a neuron-major axpy with a deterministic two-stage sum.
//
// y[b,:] = sum_j a[b,j] * W2[A_g[j], :].  The grid is (column tile, row
// chunk).  A block reads its chunk's rows over one tile of 64 16-byte vectors
// (every row slice is one coalesced 1 KB wave load), accumulates in registers,
// sums its four waves in LDS in a fixed order and writes one partial per
// (chunk, batch row, column).  A separate launch sums the chunk partials in
// chunk order and applies the merge (+ cold partial when it has active
// neurons, + b2).  No float atomics: the bits do not depend on block timing.
// (The batch-1 layer's FC2 over its group segments is in pi_fast.hip.)
#include "pi_device.h"
#include "pi_internal.h"

namespace pi {
namespace {

constexpr int kT = 256;
constexpr int kWpb = kT / kWave;
constexpr int kUnroll = 8;

template <int DT, int NBG>
__global__ __launch_bounds__(kT) void k_fc2(Fc2Args a) {
  constexpr int E = Fmt<DT>::E;
  __shared__ float red[kWpb][kWave * E];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int tile = blockIdx.x, chunk = blockIdx.y, nchunks = gridDim.y;
  const int64_t d = a.d;
  const int64_t rb = row_bytes(DT, d);
  const int nvec = (int)(rb / 16);
  const int v = tile * kWave + lane;
  const bool vok = v < nvec;
  const int vv = vok ? v : 0;
  const int64_t groups = d / 128;
  int64_t K = a.list ? (int64_t)*a.K : (int64_t)a.n_g;
  K = K < 0 ? 0 : (K > a.n_g ? a.n_g : K);
  const int64_t j0 = K * chunk / nchunks, j1 = K * (chunk + 1) / nchunks;
  const int B = a.B;
  const int64_t tile_col0 = (int64_t)tile * kWave * E;
  const char* W2 = reinterpret_cast<const char*>(a.W2);
  for (int b0 = 0; b0 < B; b0 += NBG) {
    float acc[NBG][E];
#pragma unroll
    for (int b = 0; b < NBG; ++b)
#pragma unroll
      for (int e = 0; e < E; ++e) acc[b][e] = 0.f;
    // rows j0 + wave + 4*i; the slots and activations of the next batch are read
    // while the current batch's weights are in flight
    int64_t sn[kUnroll];
    float an[kUnroll][NBG];
    auto fetch = [&](int64_t jb) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t j = jb + (int64_t)u * kWpb;
        const bool in = j < j1;
        const int64_t s = in ? (a.list ? (int64_t)a.list[j] : j) : -1;
        sn[u] = (s >= 0 && s < a.n_g) ? s : -1;
        const int64_t ai = a.a_by_row ? (sn[u] >= 0 ? sn[u] : 0) : j;
#pragma unroll
        for (int b = 0; b < NBG; ++b)
          an[u][b] = (in && sn[u] >= 0 && b0 + b < B) ? a.a[(int64_t)(b0 + b) * a.a_stride + ai] : 0.f;
      }
    };
    fetch(j0 + wave);
    for (int64_t jb = j0 + wave; jb < j1; jb += (int64_t)kWpb * kUnroll) {
      int64_t sc_[kUnroll];
      float ac[kUnroll][NBG];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        sc_[u] = sn[u];
#pragma unroll
        for (int b = 0; b < NBG; ++b) ac[u][b] = an[u][b];
      }
      uint4 w[kUnroll];
      float scl[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t s = sc_[u] >= 0 ? sc_[u] : 0;
        w[u] = sc_[u] >= 0 ? ld16(W2 + s * rb + (int64_t)vv * 16) : make_uint4(0, 0, 0, 0);
        if constexpr (DT == 2) scl[u] = sc_[u] >= 0 ? h2f(a.W2s[s * groups + vv / 4]) : 0.f;
      }
      fetch(jb + (int64_t)kWpb * kUnroll);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        float wf[E];
        widen<DT>(w[u], DT == 2 ? scl[u] : 1.f, wf);
#pragma unroll
        for (int b = 0; b < NBG; ++b)
#pragma unroll
          for (int e = 0; e < E; ++e) acc[b][e] = fmaf(ac[u][b], wf[e], acc[b][e]);
      }
    }
#pragma unroll
    for (int b = 0; b < NBG; ++b) {
      if (b0 + b < B) {
#pragma unroll
        for (int e = 0; e < E; ++e) red[wave][lane * E + e] = vok ? acc[b][e] : 0.f;
        __syncthreads();
        float* dst = a.partials + ((int64_t)chunk * B + b0 + b) * d + tile_col0;
        for (int t = tid; t < kWave * E; t += kT) {
          if (tile_col0 + t < d) {
            float sum = red[0][t];
#pragma unroll
            for (int ww = 1; ww < kWpb; ++ww) sum += red[ww][t];
            dst[t] = sum;
          }
        }
        __syncthreads();
      }
    }
  }
}

__global__ __launch_bounds__(kT) void k_reduce(ReduceArgs r) {
  const int64_t n = (int64_t)r.B * r.d;
  const bool add_c = r.y_c && (!r.K_c || *r.K_c != 0);
  for (int64_t t = blockIdx.x * (int64_t)kT + threadIdx.x; t < n; t += (int64_t)gridDim.x * kT) {
    // the cold partial and the bias are loaded with the first chunks, not after the sum
    const float yc = add_c ? r.y_c[t] : 0.f;
    const float bb = r.b2 ? load_bias(r.b2, r.b2_dt, t % r.d) : 0.f;
    float sum = 0.f;
    for (int c0 = 0; c0 < r.chunks; c0 += 16) {
      float p[16];
#pragma unroll
      for (int c = 0; c < 16; ++c) p[c] = c0 + c < r.chunks ? r.partials[(int64_t)(c0 + c) * n + t] : 0.f;
#pragma unroll
      for (int c = 0; c < 16; ++c) sum += p[c];
    }
    if (add_c) sum += yc;
    if (r.b2) sum += bb;
    r.y[t] = sum;
  }
}

// The output layer's ordered sum (as k_reduce: chunks in order, then + c2) fused
// with the activation decision: one wave per 64 ids, every batch row's logit
// stored, and the union over the batch written as the group's two words.
__global__ __launch_bounds__(kWave) void k_reduce_mask(ReduceArgs r, float tau, uint32_t* mask) {
  const int lane = threadIdx.x;
  const int64_t i = (int64_t)blockIdx.x * kWave + lane;
  const int64_t N = r.d;
  const bool in = i < N;
  const float cb = (r.b2 && in) ? load_bias(r.b2, r.b2_dt, i) : 0.f;
  bool f = false;
  for (int b0 = 0; b0 < r.B; b0 += 4) {
    float sum[4] = {0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < r.chunks; c0 += 8) {
      float p[4][8];
#pragma unroll
      for (int bb = 0; bb < 4; ++bb)
#pragma unroll
        for (int c = 0; c < 8; ++c)
          p[bb][c] = (in && b0 + bb < r.B && c0 + c < r.chunks)
                         ? r.partials[((int64_t)(c0 + c) * r.B + b0 + bb) * N + i] : 0.f;
#pragma unroll
      for (int bb = 0; bb < 4; ++bb)
#pragma unroll
        for (int c = 0; c < 8; ++c) sum[bb] += p[bb][c];
    }
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      if (in && b0 + bb < r.B) {
        float z = sum[bb];
        if (r.b2) z += cb;
        r.y[(int64_t)(b0 + bb) * N + i] = z;
        f = f || z > tau;
      }
    }
  }
  const uint64_t M = __ballot(f);
  if (lane == 0) {
    mask[2 * blockIdx.x] = (uint32_t)M;
    mask[2 * blockIdx.x + 1] = (uint32_t)(M >> 32);
  }
}

template <int DT>
hipError_t fc2_dt(const Fc2Args& a, hipStream_t s) {
  const dim3 g((unsigned)fc2_tiles(DT, a.d), (unsigned)fc2_chunks(a.B)), t(kT);
  if constexpr (DT == 2) {
    hipLaunchKernelGGL((k_fc2<DT, 1>), g, t, 0, s, a);
  } else {
    if (a.B <= 1) hipLaunchKernelGGL((k_fc2<DT, 1>), g, t, 0, s, a);
    else if (a.B <= 2) hipLaunchKernelGGL((k_fc2<DT, 2>), g, t, 0, s, a);
    else hipLaunchKernelGGL((k_fc2<DT, 4>), g, t, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

int fc2_chunks(int B) { return B <= 1 ? 64 : (B <= 2 ? 32 : (B <= 4 ? 16 : 8)); }

int fc2_tiles(int dt, int64_t d) {
  const int64_t nvec = row_bytes(dt, d) / 16;
  return (int)((nvec + kWave - 1) / kWave);
}

hipError_t launch_fc2(const Fc2Args& a, hipStream_t s) {
  switch (a.dt) {
    case PI_F32: return fc2_dt<0>(a, s);
    case PI_F16: return fc2_dt<1>(a, s);
    default: return fc2_dt<2>(a, s);
  }
}

hipError_t launch_reduce_mask(const ReduceArgs& r, float tau, uint32_t* mask, hipStream_t s) {
  hipLaunchKernelGGL(k_reduce_mask, dim3((unsigned)((r.d + kWave - 1) / kWave)), dim3(kWave), 0, s, r, tau, mask);
  return hipGetLastError();
}

hipError_t launch_reduce(const ReduceArgs& r, hipStream_t s) {
  const int64_t n = (int64_t)r.B * r.d;
  int64_t blocks = (n + kT - 1) / kT;
  blocks = blocks < 1 ? 1 : (blocks > 1024 ? 1024 : blocks);
  hipLaunchKernelGGL(k_reduce, dim3((unsigned)blocks), dim3(kT), 0, s, r);
  return hipGetLastError();
}

}  // namespace pi
