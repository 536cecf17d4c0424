// pi_fast.hip - batch-1 kernels with the input held in registers, and the
// mask + compaction epilogue shared by the fused and the batched paths.
//
// Batch-1 row dots: every lane owns the same column slice of every row
// (vectors v = u*64 + lane), so its slice of x is loaded once into VGPRs and
// reused for all the rows the wave visits.  All 16-byte loads of a row (or of
// RW rows) are issued before the first FMA.
//
// In the fused layer the output-layer kernel also emits the activation bits;
// the FC1 kernel works one 64-id block at a time from those bits and the
// prepared table, so no kernel waits on another block.
#include "pi_device.h"
#include "pi_internal.h"
#include "pi_list.h"

namespace pi {
namespace {

constexpr int kT = 256;
constexpr int kWpb = kT / kWave;
constexpr int kFc1MaxBlocks = 1024;
constexpr int kFc1T = 256;            // threads of the per-block FC1 kernel

template <int DT, int NV>
__device__ __forceinline__ void load_xreg(const float* __restrict__ x, int nvec, int lane,
                                          float (&xr)[NV][Fmt<DT>::E]) {
  constexpr int E = Fmt<DT>::E;
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int v = u * kWave + lane;
    const bool ok = v < nvec;
    const int vc = ok ? v : nvec - 1;
    const float4v* p = reinterpret_cast<const float4v*>(x + (int64_t)vc * E);
#pragma unroll
    for (int q = 0; q < E / 4; ++q) {
      const float4v t = p[q];
      xr[u][4 * q + 0] = ok ? t.x : 0.f; xr[u][4 * q + 1] = ok ? t.y : 0.f;
      xr[u][4 * q + 2] = ok ? t.z : 0.f; xr[u][4 * q + 3] = ok ? t.w : 0.f;
    }
  }
}

// The 16-byte vectors one lane reads from one row (issued together), widened and
// dotted with the lane's x slice later.
template <int DT, int NV>
struct LaneRow {
  uint4 w[NV];
  float sc[NV];
  // Branch-free and select-free: lanes past the row end read the row's last vector
  // and absent rows (rp == nullptr) read `fallback`; the caller zeroes those
  // contributions (x is zero on lanes past the row end, and an absent row's
  // result is discarded), so nothing waits on these loads before the dot product.
  __device__ __forceinline__ void issue(const char* rp, const uint16_t* sp, int nvec, int lane,
                                        const char* fallback, const uint16_t* sfallback) {
    const bool row_ok = rp != nullptr;
    const char* base = row_ok ? rp : fallback;
    const uint16_t* sbase = row_ok ? sp : sfallback;
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int v = u * kWave + lane;
      const int vc = v < nvec ? v : nvec - 1;
      w[u] = ld16(base + (int64_t)vc * 16);
      if constexpr (DT == 2) sc[u] = h2f(sbase[vc / 4]);
    }
  }
  __device__ __forceinline__ float dot(const float (&xr)[NV][Fmt<DT>::E]) const {
    constexpr int E = Fmt<DT>::E;
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      float wf[E];
      widen<DT>(w[u], DT == 2 ? sc[u] : 1.f, wf);
#pragma unroll
      for (int e = 0; e < E; ++e) acc = fmaf(wf[e], xr[u][e], acc);
    }
    return acc;
  }
};

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave)); }

// h[j] = max(0, W[j].x + bias[j]) for j < rows: one row per wave.
template <int DT, int NV, int BDT>
__global__ __launch_bounds__(kT) void k_hidden_b1(const void* __restrict__ W, const uint16_t* __restrict__ Ws,
                                                   int rows, int cols, const float* __restrict__ x,
                                                   const void* __restrict__ bias, float* __restrict__ out) {
  const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
  const int gw = blockIdx.x * kWpb + wave, nw = gridDim.x * kWpb;
  if (gw >= rows) return;
  const int64_t rb = row_bytes(DT, cols);
  const int nvec = (int)(rb / 16);
  const int groups = cols / 128;
  (void)nw;
  const Bias<BDT> bias_at(bias);
  const int j = gw;                 // the grid has one wave per row
  const float bj = bias_at(j);
  LaneRow<DT, NV> r;
  r.issue(reinterpret_cast<const char*>(W) + (int64_t)j * rb, DT == 2 ? Ws + (int64_t)j * groups : nullptr, nvec,
          lane, reinterpret_cast<const char*>(W), Ws);
  float xr[NV][Fmt<DT>::E];
  load_xreg<DT, NV>(x, nvec, lane, xr);
  float z = wave_sum(r.dot(xr)) + bj;
  z = z > 0.f ? z : 0.f;
  if (lane == 0) out[j] = z;
}

// a[j] = max(0, W1[s].x + b1[s]) (* Wup[s].x if GATED), s = list[j], j < *Kp: one row per wave.
template <int DT, int NV, bool GATED, int BDT>
__global__ __launch_bounds__(kT) void k_fc1_b1(const void* __restrict__ W, const uint16_t* __restrict__ Ws,
                                                const void* __restrict__ Wu, const uint16_t* __restrict__ Wus,
                                                int cols, const int32_t* __restrict__ list,
                                                const int32_t* __restrict__ Kp, int n_g, const float* __restrict__ x,
                                                const void* __restrict__ bias, float* __restrict__ out) {
  const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
  const int gw = blockIdx.x * kWpb + wave, nw = gridDim.x * kWpb;
  if (gw >= n_g) return;
  const int64_t rb = row_bytes(DT, cols);
  const int nvec = (int)(rb / 16);
  const int groups = cols / 128;
  (void)nw;
  const Bias<BDT> bias_at(bias);
  int K = *Kp;                       // issued with the list entry (no dependency between them)
  int s = list[gw];
  K = K < 0 ? 0 : (K > n_g ? n_g : K);
  if (gw >= K) return;
  {
    const int j = gw;                // the grid has one wave per possible list entry
    const bool ok = s >= 0 && s < n_g;
    const float bs = bias_at(ok ? s : 0);
    LaneRow<DT, NV> r, u;
    r.issue(ok ? reinterpret_cast<const char*>(W) + (int64_t)s * rb : nullptr,
            DT == 2 && ok ? Ws + (int64_t)s * groups : nullptr, nvec, lane, reinterpret_cast<const char*>(W), Ws);
    if constexpr (GATED)
      u.issue(ok ? reinterpret_cast<const char*>(Wu) + (int64_t)s * rb : nullptr,
              DT == 2 && ok ? Wus + (int64_t)s * groups : nullptr, nvec, lane, reinterpret_cast<const char*>(Wu), Wus);
    float xr[NV][Fmt<DT>::E];
    load_xreg<DT, NV>(x, nvec, lane, xr);
    float z = wave_sum(r.dot(xr)) + bs;
    z = z > 0.f ? z : 0.f;
    if constexpr (GATED) z *= wave_sum(u.dot(xr));
    if (lane == 0) out[j] = ok ? z : 0.f;
  }
}

// Position of the r-th (0-based) set bit of x (r < popcount(x)): a popcount
// descent without branches, so that no control flow separates loads that are
// in flight from their uses.
__device__ __forceinline__ int nth_set_bit64(uint64_t x, int r) {
  int base = 0;
#pragma unroll
  for (int half = 32; half >= 1; half >>= 1) {
    const uint64_t lowmask = (half == 64) ? ~0ull : ((1ull << half) - 1ull);
    const int c = __popcll(x & lowmask);
    const bool up = r >= c;
    r = up ? r - c : r;
    x = up ? (x >> half) : x;
    base = up ? base + half : base;
  }
  return base;
}

// Output layer: each wave computes 8 consecutive rows (RW at a time; for the
// usual short predictor rows all 8 rows' loads are in flight together), writes
// their logits and, with mask8 != NULL, the 8-bit activation chunk (bit k set
// when logit row0+k > tau).  One wave per 8-row group, up to a whole number
// of 64-id blocks so that every activation word is written (ids >= N are
// inactive).
template <int DT, int NV, int RW, int BDT>
__global__ __launch_bounds__(kT) void k_logits_b1(const void* __restrict__ W, const uint16_t* __restrict__ Ws, int N,
                                                   int cols, const float* __restrict__ h,
                                                   const void* __restrict__ bias,
                                                   float* __restrict__ logits, float tau, uint8_t* __restrict__ mask8) {
  const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
  const int gw = blockIdx.x * kWpb + wave, nw = gridDim.x * kWpb;
  const int ngroups = 8 * ((N + 63) / 64);
  if (gw >= ngroups) return;
  const int64_t rb = row_bytes(DT, cols);
  const int nvec = (int)(rb / 16);
  const int groups = cols / 128;
  (void)nw;
  const Bias<BDT> bias_at(bias);
  float xr[NV][Fmt<DT>::E];
  load_xreg<DT, NV>(h, nvec, lane, xr);
  {
    const int g = gw;                // the grid has one wave per 8-row group
    const int row0 = g * 8;
    // lane k < 8 holds the bias of row0 + k, read before the weights
    const float bl = bias_at(lane < 8 && row0 + lane < N ? row0 + lane : 0);
    uint32_t bits = 0;
#pragma unroll
    for (int it = 0; it < 8 / RW; ++it) {
      LaneRow<DT, NV> rr[RW];
#pragma unroll
      for (int k = 0; k < RW; ++k) {
        const int r = row0 + it * RW + k;
        const bool ok = r < N;
        rr[k].issue(ok ? reinterpret_cast<const char*>(W) + (int64_t)r * rb : nullptr,
                    DT == 2 && ok ? Ws + (int64_t)r * groups : nullptr, nvec, lane, reinterpret_cast<const char*>(W),
                    Ws);
      }
#pragma unroll
      for (int k = 0; k < RW; ++k) {
        const int r = row0 + it * RW + k;
        const float z = wave_sum(rr[k].dot(xr)) + lane_value(bl, it * RW + k);
        if (r < N) {
          if (z > tau) bits |= 1u << (it * RW + k);
          if (logits && lane == 0) logits[r] = z;
        }
      }
    }
    if (mask8 && lane == 0) mask8[g] = (uint8_t)bits;
  }
}

// FC1 of the fused batch-1 layer, one block of four waves per 64 neuron ids.
// The block's active GPU-resident neurons (activation word AND table bitmap;
// their slots from the table's per-block prefix) are spread over its waves, one
// row per wave at a time; each wave keeps x in registers, loaded after its first
// row's weights are in flight.  The block's segment receives the ascending
// slots and activations of its active GPU-resident neurons, the ascending cold
// slots of its active CPU-resident ones, and the two counts.  No block waits
// for another.
template <int DT, int NV, bool GATED, int BDT>
__global__ __launch_bounds__(kFc1T) void k_fc1_blk(const uint32_t* __restrict__ mask, SegCtx sg) {
  constexpr int WPB = kFc1T / kWave;
  const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
  const int blk = blockIdx.x;
  const uint64_t M = (uint64_t)mask[2 * blk] | ((uint64_t)mask[2 * blk + 1] << 32);
  const uint64_t G = (uint64_t)sg.gbits[2 * blk] | ((uint64_t)sg.gbits[2 * blk + 1] << 32);
  const int gp = sg.gpre[blk];
  const uint64_t act = M & G;
  const int k = __popcll(act);
  const int64_t row0 = (int64_t)blk * 64;
  if (wave == 0) {
    const uint64_t ac = M & ~G;
    const uint64_t bit = 1ull << lane, lt = bit - 1ull;
    if (ac & bit) sg.seg_cold[row0 + __popcll(ac & lt)] = (int32_t)(row0 + lane - (gp + __popcll(G & lt)));
    if (lane == 0) sg.cnt[blk] = (uint32_t)k | ((uint32_t)__popcll(ac) << 16);
  }
  if (wave >= k) return;
  const int64_t rb = row_bytes(DT, sg.d);
  const int nvec = (int)(rb / 16);
  const int groups = sg.d / 128;
  const Bias<BDT> bias_at(sg.b1);
  float xr[NV][Fmt<DT>::E];
  // the first row is peeled so that x is loaded, without a branch, right after
  // its weights are issued
  auto row = [&](int t, bool first) {
    // slot of this block's t-th active GPU-resident neuron; a table prepared
    // from another T_g cannot index past W1
    const int sl = gp + __popcll(G & ((1ull << nth_set_bit64(act, t)) - 1ull));
    const int s = sl < sg.n_g ? sl : -1;
    const float bs = bias_at(s >= 0 ? s : 0);
    LaneRow<DT, NV> r, u;
    r.issue(s >= 0 ? reinterpret_cast<const char*>(sg.W1) + (int64_t)s * rb : nullptr,
            DT == 2 && s >= 0 ? sg.W1s + (int64_t)s * groups : nullptr, nvec, lane,
            reinterpret_cast<const char*>(sg.W1), sg.W1s);
    if constexpr (GATED)
      u.issue(s >= 0 ? reinterpret_cast<const char*>(sg.Wu) + (int64_t)s * rb : nullptr,
              DT == 2 && s >= 0 ? sg.Wus + (int64_t)s * groups : nullptr, nvec, lane,
              reinterpret_cast<const char*>(sg.Wu), sg.Wus);
    if (first) load_xreg<DT, NV>(sg.x, nvec, lane, xr);
    float z = wave_sum(r.dot(xr)) + bs;
    z = z > 0.f ? z : 0.f;
    if constexpr (GATED) z *= wave_sum(u.dot(xr));
    if (lane == 0) {
      sg.seg_slot[row0 + t] = s;
      sg.seg_a[row0 + t] = s >= 0 ? z : 0.f;
    }
  };
  row(wave, true);
  for (int t = wave + WPB; t < k; t += WPB) row(t, false);
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

int grid_for(int64_t waves, int cap) {
  int64_t b = (waves + kWpb - 1) / kWpb;
  return (int)(b < 1 ? 1 : (b > cap ? cap : b));
}

template <int DT>
hipError_t hidden_dt(const B1Gemv& g, hipStream_t s) {
  const int nvec = (int)(row_bytes(DT, g.cols) / 16);
  const dim3 gr((unsigned)grid_for(g.rows, 1 << 30)), bl(kT);
#define PI_HID(NVV)                                                                                        \
  do {                                                                                                      \
    if (g.bias && g.bias_dt == 0)                                                                          \
      hipLaunchKernelGGL((k_hidden_b1<DT, NVV, 0>), gr, bl, 0, s, g.W, g.Ws, g.rows, g.cols, g.x, g.bias, g.out); \
    else                                                                                                    \
      hipLaunchKernelGGL((k_hidden_b1<DT, NVV, 1>), gr, bl, 0, s, g.W, g.Ws, g.rows, g.cols, g.x, g.bias, g.out); \
  } while (0)
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

template <int DT, bool GATED>
hipError_t fc1_dt(const B1Gemv& g, hipStream_t s) {
  const int nvec = (int)(row_bytes(DT, g.cols) / 16);
  const dim3 gr((unsigned)grid_for(g.rows, 1 << 30)), bl(kT);
#define PI_FC1(NVV)                                                                                       \
  do {                                                                                                      \
    if (g.bias && g.bias_dt == 0)                                                                          \
      hipLaunchKernelGGL((k_fc1_b1<DT, NVV, GATED, 0>), gr, bl, 0, s, g.W, g.Ws, g.Wu, g.Wus, g.cols, g.list, \
                         g.Kp, g.rows, g.x, g.bias, g.out);                                                \
    else                                                                                                    \
      hipLaunchKernelGGL((k_fc1_b1<DT, NVV, GATED, 1>), gr, bl, 0, s, g.W, g.Ws, g.Wu, g.Wus, g.cols, g.list, \
                         g.Kp, g.rows, g.x, g.bias, g.out);                                                \
  } while (0)
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
hipError_t logits_dt(const B1Gemv& g, float tau, uint8_t* mask8, hipStream_t s) {
  const int nvec = (int)(row_bytes(DT, g.cols) / 16);
  const dim3 gr((unsigned)grid_for(8 * (((int64_t)g.rows + 63) / 64), 1 << 30)), bl(kT);
#define PI_LOG(NVV, RWV)                                                                                  \
  do {                                                                                                      \
    if (g.bias && g.bias_dt == 0)                                                                          \
      hipLaunchKernelGGL((k_logits_b1<DT, NVV, RWV, 0>), gr, bl, 0, s, g.W, g.Ws, g.rows, g.cols, g.x, g.bias, \
                         g.out, tau, mask8);                                                               \
    else                                                                                                    \
      hipLaunchKernelGGL((k_logits_b1<DT, NVV, RWV, 1>), gr, bl, 0, s, g.W, g.Ws, g.rows, g.cols, g.x, g.bias, \
                         g.out, tau, mask8);                                                               \
  } while (0)
  switch (pick_nv<DT>(nvec)) {
    case 1: PI_LOG(1, 8); break;
    case 2: PI_LOG(2, 8); break;
    case 4: PI_LOG(4, 4); break;
    case 8: if constexpr (Fmt<DT>::E <= 16) PI_LOG(8, 2); break;
    case 16: if constexpr (Fmt<DT>::E <= 8) PI_LOG(16, 1); break;
    default: return hipErrorInvalidValue;
  }
#undef PI_LOG
  return hipGetLastError();
}

template <int DT, bool GATED>
hipError_t fc1_blk_dt(const uint32_t* mask, const SegCtx& sg, int nblk, hipStream_t s) {
  const int nvec = (int)(row_bytes(DT, sg.d) / 16);
  const dim3 gr((unsigned)nblk), bl(kFc1T);
  const size_t shm = 0;
#define PI_FB(NVV)                                                                    \
  do {                                                                                 \
    if (sg.b1 && sg.b1_dt == 0)                                                       \
      hipLaunchKernelGGL((k_fc1_blk<DT, NVV, GATED, 0>), gr, bl, shm, s, mask, sg);   \
    else                                                                               \
      hipLaunchKernelGGL((k_fc1_blk<DT, NVV, GATED, 1>), gr, bl, shm, s, mask, sg);   \
  } while (0)
  switch (pick_nv<DT>(nvec)) {
    case 1: PI_FB(1); break;
    case 2: PI_FB(2); break;
    case 4: PI_FB(4); break;
    case 8: if constexpr (Fmt<DT>::E <= 16) PI_FB(8); break;
    case 16: if constexpr (Fmt<DT>::E <= 8) PI_FB(16); break;
    default: return hipErrorInvalidValue;
  }
#undef PI_FB
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

hipError_t launch_fc1_b1(const B1Gemv& g, bool gated, hipStream_t s) {
  switch (g.dt) {
    case 0: return gated ? fc1_dt<0, true>(g, s) : fc1_dt<0, false>(g, s);
    case 1: return gated ? fc1_dt<1, true>(g, s) : fc1_dt<1, false>(g, s);
    default: return gated ? fc1_dt<2, true>(g, s) : fc1_dt<2, false>(g, s);
  }
}

hipError_t launch_logits_b1(const B1Gemv& g, float tau, uint8_t* mask8, hipStream_t s) {
  switch (g.dt) {
    case 0: return logits_dt<0>(g, tau, mask8, s);
    case 1: return logits_dt<1>(g, tau, mask8, s);
    default: return logits_dt<2>(g, tau, mask8, s);
  }
}

bool fc1_blk_supported(int dt, int64_t d) {
  // x staged through LDS by 512 threads x 8 float4
  return b1_supported(dt, d);
}

hipError_t launch_fc1_blk(const uint32_t* mask, const SegCtx& sg, int dtw, bool gated, int nblk, hipStream_t s) {
  switch (dtw) {
    case 0: return gated ? fc1_blk_dt<0, true>(mask, sg, nblk, s) : fc1_blk_dt<0, false>(mask, sg, nblk, s);
    case 1: return gated ? fc1_blk_dt<1, true>(mask, sg, nblk, s) : fc1_blk_dt<1, false>(mask, sg, nblk, s);
    default: return gated ? fc1_blk_dt<2, true>(mask, sg, nblk, s) : fc1_blk_dt<2, false>(mask, sg, nblk, s);
  }
}

}  // namespace pi
