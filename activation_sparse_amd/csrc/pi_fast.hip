// pi_fast.hip - batch-1 kernels with the input held in registers, and the
// mask + compaction epilogue shared by the fused and the batched paths.
//
// Batch-1 row dots: every lane owns the same column slice of every row
// (vectors v = u*64 + lane), so its slice of x is loaded once into VGPRs and
// reused for all the rows the wave visits.  All 16-byte loads of a row (or of
// RW rows) are issued before the first FMA.
//
// The output-layer kernel also emits the activation decision as bit words;
// the FC1 kernel of the fused path turns them into the active lists itself
// (pi_list.h), so no kernel waits on another block.
#include "pi_device.h"
#include "pi_internal.h"
#include "pi_list.h"

namespace pi {
namespace {

constexpr int kT = 256;
constexpr int kWpb = kT / kWave;
constexpr int kFc1MaxBlocks = 1024;

template <int DT, int NV>
__device__ __forceinline__ void load_xreg(const float* __restrict__ x, int nvec, int lane,
                                          float (&xr)[NV][Fmt<DT>::E]) {
  constexpr int E = Fmt<DT>::E;
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int v = u * kWave + lane;
    if (v < nvec) {
      const float4v* p = reinterpret_cast<const float4v*>(x + (int64_t)v * E);
#pragma unroll
      for (int q = 0; q < E / 4; ++q) {
        const float4v t = p[q];
        xr[u][4 * q + 0] = t.x; xr[u][4 * q + 1] = t.y; xr[u][4 * q + 2] = t.z; xr[u][4 * q + 3] = t.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) xr[u][e] = 0.f;
    }
  }
}

// acc[k] += dot(row k, lane's x slice) for RW rows; rp[k] == nullptr skips a row.
template <int DT, int NV, int RW>
__device__ __forceinline__ void rows_dot(const char* const (&rp)[RW], const uint16_t* const (&sp)[RW], int nvec,
                                         int lane, const float (&xr)[NV][Fmt<DT>::E], float (&acc)[RW]) {
  constexpr int E = Fmt<DT>::E;
  uint4 w[RW][NV];
#pragma unroll
  for (int k = 0; k < RW; ++k)
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int v = u * kWave + lane;
      w[k][u] = (rp[k] && v < nvec) ? ld16(rp[k] + (int64_t)v * 16) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
  for (int k = 0; k < RW; ++k)
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      float sc = 1.f;
      if constexpr (DT == 2) {
        const int v = u * kWave + lane;
        sc = (rp[k] && v < nvec) ? h2f(sp[k][v / 4]) : 0.f;
      }
      float wf[E];
      widen<DT>(w[k][u], sc, wf);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[k] = fmaf(wf[e], xr[u][e], acc[k]);
    }
}

// h[j] = max(0, W[j].x + bias[j]) for j < rows; block 0 first clears zero_n u32 words.
template <int DT, int NV>
__global__ __launch_bounds__(kT) void k_hidden_b1(const void* __restrict__ W, const uint16_t* __restrict__ Ws,
                                                   int rows, int cols, const float* __restrict__ x,
                                                   const void* __restrict__ bias, int bias_dt, float* __restrict__ out,
                                                   uint32_t* zero_ptr, int zero_n) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  if (zero_ptr && blockIdx.x == 0)
    for (int t = tid; t < zero_n; t += kT) zero_ptr[t] = 0u;
  const int64_t gw = (int64_t)blockIdx.x * kWpb + wave, nw = (int64_t)gridDim.x * kWpb;
  if (gw >= rows) return;
  const int64_t rb = row_bytes(DT, cols);
  const int nvec = (int)(rb / 16);
  float xr[NV][Fmt<DT>::E];
  load_xreg<DT, NV>(x, nvec, lane, xr);
  for (int64_t j = gw; j < rows; j += nw) {
    const char* rp[1] = {reinterpret_cast<const char*>(W) + j * rb};
    const uint16_t* sp[1] = {DT == 2 ? Ws + j * (cols / 128) : nullptr};
    float acc[1] = {0.f};
    rows_dot<DT, NV, 1>(rp, sp, nvec, lane, xr, acc);
    float z = wave_sum(acc[0]) + load_bias(bias, bias_dt, j);
    z = z > 0.f ? z : 0.f;
    if (lane == 0) out[j] = z;
  }
}

// a[j] = max(0, W1[s].x + b1[s]) (* Wup[s].x if GATED), s = list[j], j < K.
// FROM_MASK: the block first builds the lists from the activation words and
// the prepared table (writing A_g as it goes, the cold list and the counts);
// otherwise list and *Kp are inputs.
template <int DT, int NV, bool GATED, bool FROM_MASK>
__global__ __launch_bounds__(kT) void k_fc1_b1(const void* __restrict__ W, const uint16_t* __restrict__ Ws,
                                                const void* __restrict__ Wu, const uint16_t* __restrict__ Wus,
                                                int cols, const int32_t* __restrict__ list,
                                                const int32_t* __restrict__ Kp, int n_g, const float* __restrict__ x,
                                                const void* __restrict__ bias, int bias_dt, float* __restrict__ out,
                                                ListCtx lc) {
  extern __shared__ uint32_t lsm[];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  int64_t K;
  ListView lv{};
  if constexpr (FROM_MASK) {
    lv = list_build<kT>(lc, lsm);
    list_write_cold_and_counts<kT>(lc, lv);
    K = lv.K;
  } else {
    K = *Kp;
  }
  K = K < 0 ? 0 : (K > n_g ? n_g : K);
  const int64_t gw = (int64_t)blockIdx.x * kWpb + wave, nw = (int64_t)gridDim.x * kWpb;
  if (gw >= K) return;
  const int64_t rb = row_bytes(DT, cols);
  const int nvec = (int)(rb / 16);
  const int64_t groups = cols / 128;
  float xr[NV][Fmt<DT>::E];
  load_xreg<DT, NV>(x, nvec, lane, xr);
  for (int64_t j = gw; j < K; j += nw) {
    int64_t s;
    if constexpr (FROM_MASK) {
      s = list_slot(lv, (int)j);
      if (lane == 0) lc.A_g[j] = (int32_t)s;
    } else {
      s = list[j];
    }
    const bool ok = s >= 0 && s < n_g;
    const char* rp[1] = {ok ? reinterpret_cast<const char*>(W) + s * rb : nullptr};
    const uint16_t* sp[1] = {DT == 2 && ok ? Ws + s * groups : nullptr};
    float acc[1] = {0.f};
    float up[1] = {0.f};
    if constexpr (GATED) {
      const char* rq[1] = {ok ? reinterpret_cast<const char*>(Wu) + s * rb : nullptr};
      const uint16_t* sq[1] = {DT == 2 && ok ? Wus + s * groups : nullptr};
      rows_dot<DT, NV, 1>(rp, sp, nvec, lane, xr, acc);
      rows_dot<DT, NV, 1>(rq, sq, nvec, lane, xr, up);
    } else {
      rows_dot<DT, NV, 1>(rp, sp, nvec, lane, xr, acc);
    }
    float z = wave_sum(acc[0]) + (ok ? load_bias(bias, bias_dt, s) : 0.f);
    z = z > 0.f ? z : 0.f;
    if constexpr (GATED) z *= wave_sum(up[0]);
    if (lane == 0) out[j] = ok ? z : 0.f;
  }
}

}  // namespace

namespace {

// logits for 64 consecutive rows per block (16 per wave, RW at a time); with
// `mask` non-NULL also the activation words: bit i of mask[2*blk + i/32] is
// set when logit row0+i > tau.
template <int DT, int NV, int RW>
__global__ __launch_bounds__(kT) void k_logits_b1(const void* __restrict__ W, const uint16_t* __restrict__ Ws, int N,
                                                   int cols, const float* __restrict__ h,
                                                   const void* __restrict__ bias, int bias_dt,
                                                   float* __restrict__ logits, float tau, uint32_t* __restrict__ mask) {
  __shared__ float lg[64];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int64_t row0 = (int64_t)blockIdx.x * 64;
  const int64_t rb = row_bytes(DT, cols);
  const int nvec = (int)(rb / 16);
  const int64_t groups = cols / 128;
  float xr[NV][Fmt<DT>::E];
  load_xreg<DT, NV>(h, nvec, lane, xr);
  float mine = 0.f;
#pragma unroll
  for (int it = 0; it < 16 / RW; ++it) {
    const char* rp[RW];
    const uint16_t* sp[RW];
    float acc[RW];
#pragma unroll
    for (int k = 0; k < RW; ++k) {
      const int64_t r = row0 + wave * 16 + it * RW + k;
      rp[k] = r < N ? reinterpret_cast<const char*>(W) + r * rb : nullptr;
      sp[k] = (DT == 2 && r < N) ? Ws + r * groups : nullptr;
      acc[k] = 0.f;
    }
    rows_dot<DT, NV, RW>(rp, sp, nvec, lane, xr, acc);
#pragma unroll
    for (int k = 0; k < RW; ++k) {
      const int64_t r = row0 + wave * 16 + it * RW + k;
      const float t = wave_sum(acc[k]) + (r < N ? load_bias(bias, bias_dt, r) : 0.f);
      if (lane == it * RW + k) mine = t;
    }
  }
  if (lane < 16) lg[wave * 16 + lane] = mine;
  __syncthreads();
  if (wave != 0) return;
  const int64_t r = row0 + lane;
  const float v = lg[lane];
  const bool valid = r < N;
  if (logits && valid) logits[r] = v;
  if (mask) {
    const uint64_t M = __ballot(valid && v > tau);
    if (lane == 0) {
      mask[2 * blockIdx.x] = (uint32_t)M;
      mask[2 * blockIdx.x + 1] = (uint32_t)(M >> 32);
    }
  }
}

// Vectors-per-lane bound used for a row of nvec 16-byte vectors (0 = unsupported).
template <int DT>
int pick_nv(int nvec) {
  constexpr int E = Fmt<DT>::E;
  for (int nv : {1, 2, 4, 8, 16}) {
    if (nv * E > 128) break;
    if (nv * kWave >= nvec) return nv;
  }
  return 0;
}

template <int DT>
hipError_t hidden_dt(const B1Gemv& g, hipStream_t s) {
  const int nvec = (int)(row_bytes(DT, g.cols) / 16);
  int64_t blocks = (g.rows + kWpb - 1) / kWpb;
  blocks = blocks < 1 ? 1 : (blocks > 4096 ? 4096 : blocks);
  const dim3 gr((unsigned)blocks), bl(kT);
#define PI_HID(NVV) hipLaunchKernelGGL((k_hidden_b1<DT, NVV>), gr, bl, 0, s, g.W, g.Ws, g.rows, g.cols, g.x, g.bias, \
                                       g.bias_dt, g.out, g.zero_ptr, g.zero_n)
  switch (pick_nv<DT>(nvec)) {
    case 1: PI_HID(1); break;
    case 2: PI_HID(2); break;
    case 4: PI_HID(4); break;
    case 8: if constexpr (Fmt<DT>::E <= 16) PI_HID(8); break;
    case 16: if constexpr (Fmt<DT>::E <= 8) PI_HID(16); break;
    default: return hipErrorInvalidValue;
  }
#undef PI_HID
  return hipGetLastError();
}

template <int DT, bool GATED, bool FM>
hipError_t fc1_dt(const B1Gemv& g, const ListCtx& lc, hipStream_t s) {
  const int nvec = (int)(row_bytes(DT, g.cols) / 16);
  int64_t blocks = (g.rows + kWpb - 1) / kWpb;   // rows = n_g (bound on K)
  blocks = blocks < 1 ? 1 : (blocks > kFc1MaxBlocks ? kFc1MaxBlocks : blocks);
  const dim3 gr((unsigned)blocks), bl(kT);
  const size_t shm = FM ? (size_t)list_smem_words(lc.W) * 4 : 0;
#define PI_FC1(NVV) hipLaunchKernelGGL((k_fc1_b1<DT, NVV, GATED, FM>), gr, bl, shm, s, g.W, g.Ws, g.Wu, g.Wus, g.cols, \
                                       g.list, g.Kp, g.rows, g.x, g.bias, g.bias_dt, g.out, lc)
  switch (pick_nv<DT>(nvec)) {
    case 1: PI_FC1(1); break;
    case 2: PI_FC1(2); break;
    case 4: PI_FC1(4); break;
    case 8: if constexpr (Fmt<DT>::E <= 16) PI_FC1(8); break;
    case 16: if constexpr (Fmt<DT>::E <= 8) PI_FC1(16); break;
    default: return hipErrorInvalidValue;
  }
#undef PI_FC1
  return hipGetLastError();
}

template <int DT>
hipError_t logits_dt(const B1Gemv& g, float tau, uint32_t* mask, hipStream_t s) {
  const int nvec = (int)(row_bytes(DT, g.cols) / 16);
  const dim3 gr((unsigned)((g.rows + 63) / 64)), bl(kT);
#define PI_LOG(NVV, RWV) hipLaunchKernelGGL((k_logits_b1<DT, NVV, RWV>), gr, bl, 0, s, g.W, g.Ws, g.rows, \
                                            g.cols, g.x, g.bias, g.bias_dt, g.out, tau, mask)
  switch (pick_nv<DT>(nvec)) {
    case 1: PI_LOG(1, 16); break;
    case 2: PI_LOG(2, 16); break;
    case 4: PI_LOG(4, 8); break;
    case 8: if constexpr (Fmt<DT>::E <= 16) PI_LOG(8, 4); break;
    case 16: if constexpr (Fmt<DT>::E <= 8) PI_LOG(16, 2); break;
    default: return hipErrorInvalidValue;
  }
#undef PI_LOG
  return hipGetLastError();
}

}  // namespace

bool b1_supported(int dt, int64_t cols) {
  const int nvec = (int)(row_bytes(dt, cols) / 16);
  switch (dt) {
    case 0: return pick_nv<0>(nvec) != 0;
    case 1: return pick_nv<1>(nvec) != 0;
    default: return pick_nv<2>(nvec) != 0;
  }
}

hipError_t launch_hidden_b1(const B1Gemv& g, hipStream_t s) {
  switch (g.dt) {
    case 0: return hidden_dt<0>(g, s);
    case 1: return hidden_dt<1>(g, s);
    default: return hidden_dt<2>(g, s);
  }
}

template <int DT>
hipError_t fc1_dt2(const B1Gemv& g, bool gated, const ListCtx* lc, hipStream_t s) {
  if (lc) return gated ? fc1_dt<DT, true, true>(g, *lc, s) : fc1_dt<DT, false, true>(g, *lc, s);
  const ListCtx none{};
  return gated ? fc1_dt<DT, true, false>(g, none, s) : fc1_dt<DT, false, false>(g, none, s);
}

hipError_t launch_fc1_b1(const B1Gemv& g, bool gated, const ListCtx* lc, hipStream_t s) {
  switch (g.dt) {
    case 0: return fc1_dt2<0>(g, gated, lc, s);
    case 1: return fc1_dt2<1>(g, gated, lc, s);
    default: return fc1_dt2<2>(g, gated, lc, s);
  }
}

hipError_t launch_logits_b1(const B1Gemv& g, float tau, uint32_t* mask, hipStream_t s) {
  switch (g.dt) {
    case 0: return logits_dt<0>(g, tau, mask, s);
    case 1: return logits_dt<1>(g, tau, mask, s);
    default: return logits_dt<2>(g, tau, mask, s);
  }
}

}  // namespace pi
