// pi_fc2.hip - FC2 as a neuron-major axpy with a deterministic two-stage sum.
//
// y[b,:] = sum_j a[b,j] * W2[A_g[j], :].  The grid is (column tile, row
// chunk).  A block reads its chunk's rows over one tile of 64 16-byte vectors
// (every row slice is one coalesced 1 KB wave load), accumulates in registers,
// sums its four waves in LDS in a fixed order and writes one partial per
// (chunk, batch row, column).  The last block to finish a column tile (tile
// counter) sums the chunk partials in chunk order and applies the merge
// (+ cold partial when it has active neurons, + b2).  No float atomics: the
// bits do not depend on block timing.
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
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int tile = blockIdx.x, chunk = blockIdx.y, nchunks = gridDim.y;
  const int64_t d = a.d;
  const int64_t rb = row_bytes(DT, d);
  const int nvec = (int)(rb / 16);
  const int v = tile * kWave + lane;
  const bool vok = v < nvec;
  const int64_t groups = d / 128;
  int64_t K = *a.K;
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
    for (int64_t jb = j0 + wave; jb < j1; jb += (int64_t)kWpb * kUnroll) {
      int64_t s[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t j = jb + (int64_t)u * kWpb;
        s[u] = j < j1 ? (int64_t)a.list[j] : -1;
        if (s[u] >= a.n_g) s[u] = -1;
      }
      uint4 w[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        w[u] = (s[u] >= 0 && vok) ? ld16(W2 + s[u] * rb + (int64_t)v * 16) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (s[u] < 0) continue;
        const int64_t j = jb + (int64_t)u * kWpb;
        float sc = 1.f;
        if constexpr (DT == 2) sc = vok ? h2f(a.W2s[s[u] * groups + v / 4]) : 0.f;
        float wf[E];
        widen<DT>(w[u], sc, wf);
#pragma unroll
        for (int b = 0; b < NBG; ++b) {
          if (b0 + b < B) {
            const float ab = a.a[(int64_t)(b0 + b) * a.n_g + j];
#pragma unroll
            for (int e = 0; e < E; ++e) acc[b][e] = fmaf(ab, wf[e], acc[b][e]);
          }
        }
      }
    }
#pragma unroll
    for (int b = 0; b < NBG; ++b) {
      if (b0 + b < B) {
#pragma unroll
        for (int e = 0; e < E; ++e) red[wave][lane * E + e] = acc[b][e];
        __syncthreads();
        float* dst = a.partials + ((int64_t)chunk * B + b0 + b) * d + tile_col0;
        for (int t = tid; t < kWave * E; t += kT) {
          if (tile_col0 + t < d) {
            float sum = red[0][t];
#pragma unroll
            for (int w = 1; w < kWpb; ++w) sum += red[w][t];
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
    float sum = 0.f;
#pragma unroll 8
    for (int c = 0; c < r.chunks; ++c) sum += r.partials[(int64_t)c * n + t];
    if (add_c) sum += r.y_c[t];
    if (r.b2) sum += load_bias(r.b2, r.b2_dt, t % r.d);
    r.y[t] = sum;
  }
}

template <int DT>
hipError_t fc2_dt(const Fc2Args& a, hipStream_t s) {
  const dim3 g((unsigned)fc2_tiles(DT, a.d), (unsigned)kFc2Chunks), t(kT);
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

hipError_t launch_reduce(const ReduceArgs& r, hipStream_t s) {
  const int64_t n = (int64_t)r.B * r.d;
  int64_t blocks = (n + kT - 1) / kT;
  blocks = blocks < 1 ? 1 : (blocks > 1024 ? 1024 : blocks);
  hipLaunchKernelGGL(k_reduce, dim3((unsigned)blocks), dim3(kT), 0, s, r);
  return hipGetLastError();
}

}  // namespace pi
