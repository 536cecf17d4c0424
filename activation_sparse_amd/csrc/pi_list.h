// pi_list.h - active lists from activation bit words and the prepared table.
//
// Every block that needs the lists rebuilds them from two small arrays of W
// 32-bit words (the activation decision of each neuron id, and the bitmap of
// GPU-resident ids from the prepared neuron table): one coalesced load of the
// words, three block-wide exclusive scans of their popcounts, and a binary
// search per list position.  The list of GPU-resident active neurons is the
// ascending run of their slots (the rank of an id among the GPU-resident
// ids); the CPU list the ascending run of cold slots (the rank among the
// others).  No block waits for another.
#pragma once
#include "pi_device.h"

namespace pi {

struct ListCtx {
  const uint32_t* mask;   // [W] activation words
  const uint32_t* gbits;  // [W] GPU-resident bitmap
  int W;                  // words (covers all N ids; bits >= N are zero in both)
  int32_t* A_g;
  int32_t* K;
  int32_t* A_c;           // NULL = no cold list
  int32_t* K_c;
  int32_t* rows_read;     // optional: [1] = K, and [0] = rows0 when rows0 >= 0
  int32_t rows0;
};

// LDS words needed by list_build for W words.
__host__ __device__ constexpr int list_smem_words(int W) { return 6 * W + 4; }

struct ListView {
  const uint32_t* act;    // [W] active GPU-resident bits
  const uint32_t* gw;     // [W] GPU-resident bits
  const uint32_t* cold;   // [W] active CPU-resident bits
  const int32_t* pact;    // [W+1] exclusive prefix of popc(act)
  const int32_t* pg;      // [W+1] exclusive prefix of popc(gw)
  const int32_t* pcold;   // [W+1] exclusive prefix of popc(cold)
  int W;
  int K, Kc;
};

__device__ __forceinline__ int nth_set_bit(uint32_t x, int r) {
  for (int i = 0; i < r; ++i) x &= x - 1u;
  return __builtin_ctz(x);
}

// Largest w with p[w] <= j, for p non-decreasing over [0, W] and p[W] > j.
__device__ __forceinline__ int upper_word(const int32_t* p, int W, int j) {
  int lo = 0, hi = W;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p[mid] <= j) lo = mid; else hi = mid;
  }
  return lo;
}

// Slot (rank among GPU-resident ids) of list position j < K.
__device__ __forceinline__ int list_slot(const ListView& v, int j) {
  const int w = upper_word(v.pact, v.W, j);
  const int bit = nth_set_bit(v.act[w], j - v.pact[w]);
  return v.pg[w] + __popc(v.gw[w] & ((1u << bit) - 1u));
}

// Cold slot (rank among the other ids) of cold list position j < Kc.
__device__ __forceinline__ int list_cold_slot(const ListView& v, int j) {
  const int w = upper_word(v.pcold, v.W, j);
  const int bit = nth_set_bit(v.cold[w], j - v.pcold[w]);
  const int id = 32 * w + bit;
  return id - (v.pg[w] + __popc(v.gw[w] & ((1u << bit) - 1u)));
}

// Block-wide build (all NT threads call it); sm has list_smem_words(W) words.
template <int NT>
__device__ ListView list_build(const ListCtx& c, uint32_t* sm) {
  constexpr int NW = NT / kWave;
  const int W = c.W;
  uint32_t* act = sm;
  uint32_t* gw = act + W;
  uint32_t* cold = gw + W;
  int32_t* pact = reinterpret_cast<int32_t*>(cold + W);
  int32_t* pg = pact + (W + 1);
  int32_t* pcold = pg + (W + 1);
  __shared__ int wsum[3][NW];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  const int per = (W + NT - 1) / NT;
  const int w0 = tid * per;
  int sa = 0, sg = 0, sc = 0;
  for (int k = 0; k < per; ++k) {
    const int w = w0 + k;
    if (w < W) {
      const uint32_t m = c.mask[w], g = c.gbits[w];
      const uint32_t a = m & g, cl = m & ~g;
      act[w] = a; gw[w] = g; cold[w] = cl;
      sa += __popc(a); sg += __popc(g); sc += __popc(cl);
    }
  }
  // block exclusive scan of (sa, sg, sc) over threads in order
  int ia = sa, ig = sg, ic = sc;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int ta = __shfl_up(ia, off, kWave), tg = __shfl_up(ig, off, kWave), tc = __shfl_up(ic, off, kWave);
    if (lane >= off) { ia += ta; ig += tg; ic += tc; }
  }
  if (lane == kWave - 1) { wsum[0][wv] = ia; wsum[1][wv] = ig; wsum[2][wv] = ic; }
  __syncthreads();
  int ba = 0, bg = 0, bc = 0, ta = 0, tg = 0, tc = 0;
  for (int w = 0; w < NW; ++w) {
    if (w < wv) { ba += wsum[0][w]; bg += wsum[1][w]; bc += wsum[2][w]; }
    ta += wsum[0][w]; tg += wsum[1][w]; tc += wsum[2][w];
  }
  int ra = ba + ia - sa, rg = bg + ig - sg, rc = bc + ic - sc;
  for (int k = 0; k < per; ++k) {
    const int w = w0 + k;
    if (w < W) {
      pact[w] = ra; pg[w] = rg; pcold[w] = rc;
      ra += __popc(act[w]); rg += __popc(gw[w]); rc += __popc(cold[w]);
    }
  }
  if (tid == 0) { pact[W] = ta; pg[W] = tg; pcold[W] = tc; }
  __syncthreads();
  ListView v{act, gw, cold, pact, pg, pcold, W, ta, tc};
  return v;
}

// Writes the cold list (block-strided over positions) and, from block 0, the counts.
template <int NT>
__device__ void list_write_cold_and_counts(const ListCtx& c, const ListView& v) {
  if (c.A_c)
    for (int j = blockIdx.x * NT + threadIdx.x; j < v.Kc; j += gridDim.x * NT) c.A_c[j] = list_cold_slot(v, j);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    *c.K = v.K;
    if (c.K_c) *c.K_c = v.Kc;
    if (c.rows_read) {
      if (c.rows0 >= 0) c.rows_read[0] = c.rows0;
      c.rows_read[1] = v.K;
    }
  }
}

}  // namespace pi
