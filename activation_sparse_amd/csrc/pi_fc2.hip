// pi_fc2.hip - FC2 as a neuron-major axpy with a deterministic two-stage sum.
//
// y[b,:] = sum_j a[b,j] * W2[A_g[j], :].  The grid is (column tile, row
// chunk).  A block reads its chunk's rows over one tile of 64 16-byte vectors
// (every row slice is one coalesced 1 KB wave load), accumulates in registers,
// sums its four waves in LDS in a fixed order and writes one partial per
// (chunk, batch row, column).  A separate launch sums the chunk partials in
// chunk order and applies the merge (+ cold partial when it has active
// neurons, + b2).  No float atomics: the bits do not depend on block timing.
#include "pi_device.h"
#include "pi_internal.h"

namespace pi {
namespace {

constexpr int kT = 256;
constexpr int kWpb = kT / kWave;
constexpr int kUnroll = 8;
constexpr int kSegUnroll = 16;

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
    float sum = 0.f;
    for (int c0 = 0; c0 < r.chunks; c0 += 16) {
      float p[16];
#pragma unroll
      for (int c = 0; c < 16; ++c) p[c] = c0 + c < r.chunks ? r.partials[(int64_t)(c0 + c) * n + t] : 0.f;
#pragma unroll
      for (int c = 0; c < 16; ++c) sum += p[c];
    }
    if (add_c) sum += r.y_c[t];
    if (r.b2) sum += load_bias(r.b2, r.b2_dt, t % r.d);
    r.y[t] = sum;
  }
}

// Batch-1 FC2 over the group segments of the fused layer, and the list
// assembly.  Blocks [0, tiles * kSegChunks) are FC2 blocks: block (tile,
// chunk) takes the groups [c * ngroups / C, (c + 1) * ngroups / C); its rows are
// those groups' (slot, a) pairs with a != 0 in group order (ascending slots),
// gathered into LDS first (one round trip), then the listed W2 rows are
// streamed over the block's column tile: 16-byte loads, kSegUnroll rows in
// flight per wave.  It writes one partial per chunk.  The other blocks each
// place 256 entries (four groups) of the ascending lists A_g / A_c, at offsets
// from the counts of the groups below; list block 0 writes K and K_c.
template <int DT>
__global__ __launch_bounds__(kT) void k_fc2_seg(Fc2SegArgs a, int tiles) {
  constexpr int E = Fmt<DT>::E;
  extern __shared__ int32_t fsm[];
  __shared__ float red[kWpb][kWave * E];
  __shared__ int s_cnt[64], s_off[65];
  __shared__ int s_red[5][kWpb];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int ngroups = a.ngroups;
  if ((int)blockIdx.x >= tiles * kSegChunks) {
    // ---- list assembly: groups [4 lb, 4 lb + 4), one entry per thread
    const int lb = (int)blockIdx.x - tiles * kSegChunks;
    const int g0 = 4 * lb;
    const int e = g0 * 64 + tid;
    const int grp = e / 64, i = e % 64;
    const bool ein = grp < ngroups;
    const int32_t es = ein ? a.seg_slot[e] : 0;
    const int32_t ec = (ein && a.A_c) ? a.seg_cold[e] : 0;
    const uint32_t mine = ein ? a.cnt[grp] : 0u;
    // counts below g0 and in total, summed over a strided share of the groups
    int below_g = 0, below_c = 0, tot_g = 0, tot_c = 0, tot_z = 0;
    for (int q = tid; q < ngroups; q += kT) {
      const uint32_t c = a.cnt[q];
      const int cg = (int)cnt_gpu(c), cc = (int)cnt_cold(c);
      tot_g += cg; tot_c += cc; tot_z += (int)cnt_nz(c);
      if (q < g0) { below_g += cg; below_c += cc; }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      below_g += __shfl_xor(below_g, off, kWave); below_c += __shfl_xor(below_c, off, kWave);
      tot_g += __shfl_xor(tot_g, off, kWave); tot_c += __shfl_xor(tot_c, off, kWave);
      tot_z += __shfl_xor(tot_z, off, kWave);
    }
    if (lane == 0) {
      s_red[0][wave] = below_g; s_red[1][wave] = below_c; s_red[2][wave] = tot_g; s_red[3][wave] = tot_c;
      s_red[4][wave] = tot_z;
    }
    if (lane == 0 && wave < 4) s_cnt[wave] = g0 + wave < ngroups ? (int)a.cnt[g0 + wave] : 0;
    __syncthreads();
    int bg = 0, bc = 0, tg = 0, tc = 0, tz = 0;
#pragma unroll
    for (int w = 0; w < kWpb; ++w) {
      bg += s_red[0][w]; bc += s_red[1][w]; tg += s_red[2][w]; tc += s_red[3][w]; tz += s_red[4][w];
    }
    // offsets of this thread's group within the block's four
    const int gi = tid / 64;
    for (int w = 0; w < gi; ++w) { bg += (int)cnt_gpu((uint32_t)s_cnt[w]); bc += (int)cnt_cold((uint32_t)s_cnt[w]); }
    if (ein && i < (int)cnt_gpu(mine) && bg + i < a.n_g) a.A_g[bg + i] = es;
    if (ein && a.A_c && i < (int)cnt_cold(mine) && bc + i < a.n_c) a.A_c[bc + i] = ec;
    if (lb == 0 && tid == 0) {
      *a.K = tg < a.n_g ? tg : a.n_g;
      if (a.K_c) *a.K_c = tc < a.n_c ? tc : a.n_c;
      if (a.rows_read) *a.rows_read = tz;
    }
    return;
  }
  // ---- FC2
  const int tile = (int)blockIdx.x % tiles, chunk = (int)blockIdx.x / tiles;
  const int b0 = (int)((int64_t)ngroups * chunk / kSegChunks), b1 = (int)((int64_t)ngroups * (chunk + 1) / kSegChunks);
  const int nb = b1 - b0;
  int32_t* c_slot = fsm;
  float* c_a = reinterpret_cast<float*>(fsm + nb * 64);
  // each thread's share of the raw (slot, a) entries, loaded together with the counts
  constexpr int RQ = 16;   // entries per thread: nb * 64 <= RQ * kT
  int32_t rs[RQ];
  float ra[RQ];
#pragma unroll
  for (int q = 0; q < RQ; ++q) {
    const int e = q * kT + tid;
    rs[q] = e < nb * 64 ? a.pos_slot[(int64_t)b0 * 64 + e] : -1;
    ra[q] = e < nb * 64 ? a.pos_a[(int64_t)b0 * 64 + e] : 0.f;
  }
  if (tid < nb) s_cnt[tid] = (int)cnt_nz(a.cnt[b0 + tid]);
  __syncthreads();
  if (wave == 0) {
    const int v = lane < nb ? s_cnt[lane] : 0;
    int incl = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int t = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += t;
    }
    if (lane < nb) s_off[lane] = incl - v;
    if (lane == kWave - 1) s_off[nb] = incl;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < RQ; ++q) {
    const int e = q * kT + tid;
    if (e < nb * 64) {
      const int bb = e / 64, i = e % 64;
      if (i < s_cnt[bb]) {
        c_slot[s_off[bb] + i] = rs[q];
        c_a[s_off[bb] + i] = ra[q];
      }
    }
  }
  __syncthreads();
  const int R = s_off[nb];
  const int64_t d = a.d;
  const int64_t rb = row_bytes(DT, d);
  const int nvec = (int)(rb / 16);
  const int v = tile * kWave + lane;
  const bool vok = v < nvec;
  const int64_t groups = d / 128;
  const int64_t tile_col0 = (int64_t)tile * kWave * E;
  const char* W2 = reinterpret_cast<const char*>(a.W2);
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int jb = wave; jb < R; jb += kWpb * kSegUnroll) {
    uint4 w[kSegUnroll];
    float scl[kSegUnroll], ab[kSegUnroll];
#pragma unroll
    for (int u = 0; u < kSegUnroll; ++u) {
      // row j is the same for the whole wave: a buffer over it, empty for an
      // absent row; lanes past the row end read zeros
      const int j = jb + u * kWpb;
      int s = j < R ? c_slot[j] : -1;
      s = __builtin_amdgcn_readfirstlane(s < a.n_g ? s : -1);
      ab[u] = j < R ? c_a[j] : 0.f;
      const rsrc_t rw = make_rsrc(W2 + (s >= 0 ? (int64_t)s * rb : 0), s >= 0 ? (uint32_t)rb : 0u);
      w[u] = bload16(rw, (uint32_t)v * 16u);
      if constexpr (DT == 2) {
        const rsrc_t rs = make_rsrc(a.W2s + (s >= 0 ? (int64_t)s * groups : 0), s >= 0 ? (uint32_t)groups * 2u : 0u);
        scl[u] = h2f(bload2(rs, (uint32_t)(v / 4) * 2u));
      }
    }
#pragma unroll
    for (int u = 0; u < kSegUnroll; ++u) {
      float wf[E];
      widen<DT>(w[u], DT == 2 ? scl[u] : 1.f, wf);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = fmaf(ab[u], wf[e], acc[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) red[wave][lane * E + e] = vok ? acc[e] : 0.f;
  __syncthreads();
  float* dst = a.partials + (int64_t)chunk * d + tile_col0;
  for (int t = tid; t < kWave * E; t += kT) {
    if (tile_col0 + t < d) {
      float sum = red[0][t];
#pragma unroll
      for (int ww = 1; ww < kWpb; ++ww) sum += red[ww][t];
      dst[t] = sum;
    }
  }
}

// y[t] = the kSegChunks partials summed in chunk order (+ y_c when K_c is NULL
// or *K_c != 0, + b2): one column per thread, every partial load in flight.
__global__ __launch_bounds__(kWave) void k_reduce_y(ReduceYArgs r) {
  const int64_t t = (int64_t)blockIdx.x * kWave + threadIdx.x;
  if (t >= r.d) return;
  const int kc = r.K_c ? *r.K_c : 1;
  const float yc = r.y_c ? r.y_c[t] : 0.f;
  const float bb = r.b2 ? load_bias(r.b2, r.b2_dt, t) : 0.f;
  float p[kSegChunks];
#pragma unroll
  for (int c = 0; c < kSegChunks; ++c) p[c] = r.partials[(int64_t)c * r.d + t];
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < kSegChunks; ++c) sum += p[c];
  if (r.y_c && kc != 0) sum += yc;
  if (r.b2) sum += bb;
  r.y[t] = sum;
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

hipError_t launch_fc2_seg(const Fc2SegArgs& a, hipStream_t s) {
  const int nbmax = (a.ngroups + kSegChunks - 1) / kSegChunks;
  const size_t shm = (size_t)nbmax * 64 * 4 * 2;
  const int tiles = fc2_tiles(a.dt, a.d);
  const int list_blocks = (a.ngroups + 3) / 4;
  const dim3 g((unsigned)(tiles * kSegChunks + list_blocks)), t(kT);
  switch (a.dt) {
    case PI_F32: hipLaunchKernelGGL(k_fc2_seg<0>, g, t, shm, s, a, tiles); break;
    case PI_F16: hipLaunchKernelGGL(k_fc2_seg<1>, g, t, shm, s, a, tiles); break;
    default: hipLaunchKernelGGL(k_fc2_seg<2>, g, t, shm, s, a, tiles); break;
  }
  return hipGetLastError();
}

hipError_t launch_reduce_y(const ReduceYArgs& r, hipStream_t s) {
  hipLaunchKernelGGL(k_reduce_y, dim3((unsigned)((r.d + kWave - 1) / kWave)), dim3(kWave), 0, s, r);
  return hipGetLastError();
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
