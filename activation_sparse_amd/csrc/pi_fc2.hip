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
constexpr int kSegUnroll = 8;

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
    // rows j0 + wave + 4*i; the slots and activations of the next batch are read
    // while the current batch's weights are in flight
    int64_t sn[kUnroll];
    float an[kUnroll][NBG];
    auto fetch = [&](int64_t jb) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t j = jb + (int64_t)u * kWpb;
        const bool in = j < j1;
        const int64_t s = in ? (int64_t)a.list[j] : -1;
        sn[u] = (s >= 0 && s < a.n_g) ? s : -1;
#pragma unroll
        for (int b = 0; b < NBG; ++b) an[u][b] = (in && b0 + b < B) ? a.a[(int64_t)(b0 + b) * a.n_g + j] : 0.f;
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

// Batch-1 FC2 over the per-64-id-block segments of the fused layer: chunk c
// covers the blocks [c*nblk/C, (c+1)*nblk/C); its rows are those blocks'
// active GPU-resident neurons in block order (so in ascending slot order).
// The block's segment entries are gathered into LDS first (one round trip).
template <int DT>
__global__ __launch_bounds__(kT) void k_fc2_seg(Fc2SegArgs a) {
  constexpr int E = Fmt<DT>::E;
  extern __shared__ int32_t fsm[];
  __shared__ float red[kWpb][kWave * E];
  __shared__ int s_cnt[64], s_off[65];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int tile = blockIdx.x, chunk = blockIdx.y, nchunks = gridDim.y;
  const int b0 = (int)((int64_t)a.nblk * chunk / nchunks), b1 = (int)((int64_t)a.nblk * (chunk + 1) / nchunks);
  const int nb = b1 - b0;
  int32_t* c_slot = fsm;
  float* c_a = reinterpret_cast<float*>(fsm + nb * 64);
  // each thread's share of the raw segment entries, loaded together with the counts
  constexpr int RQ = 16;   // entries per thread: nb * 64 <= RQ * kT
  int32_t rs[RQ];
  float ra[RQ];
#pragma unroll
  for (int q = 0; q < RQ; ++q) {
    const int e = q * kT + tid;
    rs[q] = e < nb * 64 ? a.seg_slot[(int64_t)b0 * 64 + e] : -1;
    ra[q] = e < nb * 64 ? a.seg_a[(int64_t)b0 * 64 + e] : 0.f;
  }
  if (tid < nb) s_cnt[tid] = (int)(a.cnt[b0 + tid] & 0xFFFFu);
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
  const int vv = vok ? v : 0;
  const int64_t groups = d / 128;
  const int64_t tile_col0 = (int64_t)tile * kWave * E;
  const char* W2 = reinterpret_cast<const char*>(a.W2);
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int jb = wave; jb < R; jb += kWpb * kUnroll) {
    int64_t sl[kUnroll];
    uint4 w[kUnroll];
    float scl[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int j = jb + u * kWpb;
      int64_t s = j < R ? (int64_t)c_slot[j] : -1;
      if (s >= a.n_g) s = -1;
      sl[u] = s;
      const int64_t s0 = s >= 0 ? s : 0;
      w[u] = s >= 0 ? ld16(W2 + s0 * rb + (int64_t)vv * 16) : make_uint4(0, 0, 0, 0);
      if constexpr (DT == 2) scl[u] = s >= 0 ? h2f(a.W2s[s0 * groups + vv / 4]) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (sl[u] < 0) continue;
      float wf[E];
      widen<DT>(w[u], DT == 2 ? scl[u] : 1.f, wf);
      const float ab = c_a[jb + u * kWpb];
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = fmaf(ab, wf[e], acc[e]);
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

// Exclusive scans of two count arrays into LDS; returns the totals.
__device__ void block_scan2(const int* c1, const int* c2, int n, int* o1, int* o2, int& t1, int& t2) {
  __shared__ int ws1[kWpb], ws2[kWpb];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  const int per = (n + kT - 1) / kT, i0 = tid * per;
  int s1 = 0, s2 = 0;
  for (int k = 0; k < per; ++k)
    if (i0 + k < n) { s1 += c1[i0 + k]; s2 += c2[i0 + k]; }
  int a1 = s1, a2 = s2;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int u1 = __shfl_up(a1, off, kWave), u2 = __shfl_up(a2, off, kWave);
    if (lane >= off) { a1 += u1; a2 += u2; }
  }
  if (lane == kWave - 1) { ws1[wv] = a1; ws2[wv] = a2; }
  __syncthreads();
  int p1 = 0, p2 = 0;
  t1 = 0; t2 = 0;
  for (int w = 0; w < kWpb; ++w) {
    if (w < wv) { p1 += ws1[w]; p2 += ws2[w]; }
    t1 += ws1[w]; t2 += ws2[w];
  }
  int r1 = p1 + a1 - s1, r2 = p2 + a2 - s2;
  for (int k = 0; k < per; ++k)
    if (i0 + k < n) { o1[i0 + k] = r1; o2[i0 + k] = r2; r1 += c1[i0 + k]; r2 += c2[i0 + k]; }
  __syncthreads();
}

// Blocks [0, reduce_blocks): y = ordered sum of the FC2 partials (+ cold partial
// when the cold side has an active neuron, + b2).  The other blocks assemble
// the ascending lists A_g / A_c from the segments, 256 entries each; the first
// of them writes K and K_c.
__global__ __launch_bounds__(kT) void k_reduce_lists(ReduceListArgs r) {
  extern __shared__ int rsm[];
  const int tid = threadIdx.x;
  const int nblk = r.nblk;
  if ((int)blockIdx.x < r.reduce_blocks) {
    __shared__ int any_cold;
    if (tid == 0) any_cold = 0;
    __syncthreads();
    bool mine = false;
    if (r.y_c && !r.always_c)
      for (int b = tid; b < nblk; b += kT) mine = mine || (r.cnt[b] >> 16) != 0u;
    if (mine) any_cold = 1;
    __syncthreads();
    const bool add_c = r.y_c && (r.always_c || any_cold);
    const int64_t n = r.d;
    for (int64_t t = blockIdx.x * (int64_t)kT + tid; t < n; t += (int64_t)r.reduce_blocks * kT) {
      float sum = 0.f;
      for (int c0 = 0; c0 < r.chunks; c0 += 16) {
        float p[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) p[c] = c0 + c < r.chunks ? r.partials[(int64_t)(c0 + c) * n + t] : 0.f;
#pragma unroll
        for (int c = 0; c < 16; ++c) sum += p[c];
      }
      if (add_c) sum += r.y_c[t];
      if (r.b2) sum += load_bias(r.b2, r.b2_dt, t);
      r.y[t] = sum;
    }
    return;
  }
  const int lb = (int)blockIdx.x - r.reduce_blocks;
  int* cg = rsm;
  int* cc = rsm + nblk;
  int* og = rsm + 2 * nblk;
  int* oc = rsm + 3 * nblk;
  // this block's entries: 4 id blocks x 64 = 256, one per thread, loaded with the counts
  const int e = lb * kT + tid;
  const bool ein = e < nblk * 64;
  const int32_t es = ein ? r.seg_slot[e] : 0;
  const int32_t ec = (ein && r.A_c) ? r.seg_cold[e] : 0;
  for (int b = tid; b < nblk; b += kT) {
    const uint32_t c = r.cnt[b];
    cg[b] = (int)(c & 0xFFFFu);
    cc[b] = (int)(c >> 16);
  }
  __syncthreads();
  int tg, tc;
  block_scan2(cg, cc, nblk, og, oc, tg, tc);
  if (ein) {
    const int b = e / 64, i = e % 64;
    if (i < cg[b] && og[b] + i < r.n_g) r.A_g[og[b] + i] = es;
    if (r.A_c && i < cc[b] && oc[b] + i < r.n_c) r.A_c[oc[b] + i] = ec;
  }
  if (lb == 0 && tid == 0) {
    *r.K = tg < r.n_g ? tg : r.n_g;
    if (r.K_c) *r.K_c = tc < r.n_c ? tc : r.n_c;
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
  const int nbmax = (a.nblk + kSegChunks - 1) / kSegChunks;
  const size_t shm = (size_t)nbmax * 64 * 4 * 2;
  const dim3 g((unsigned)fc2_tiles(a.dt, a.d), (unsigned)kSegChunks), t(kT);
  switch (a.dt) {
    case PI_F32: hipLaunchKernelGGL(k_fc2_seg<0>, g, t, shm, s, a); break;
    case PI_F16: hipLaunchKernelGGL(k_fc2_seg<1>, g, t, shm, s, a); break;
    default: hipLaunchKernelGGL(k_fc2_seg<2>, g, t, shm, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_reduce_lists(const ReduceListArgs& r, hipStream_t s) {
  const int list_blocks = (int)(((int64_t)r.nblk * 64 + kT - 1) / kT);
  ReduceListArgs q = r;
  q.reduce_blocks = (int)((r.d + kT - 1) / kT);
  q.chunks = kSegChunks;
  hipLaunchKernelGGL(k_reduce_lists, dim3((unsigned)(q.reduce_blocks + list_blocks)), dim3(kT),
                     (size_t)r.nblk * 4 * 4, s, q);
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
