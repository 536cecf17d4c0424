// pi_b1_dev.h - device pieces of the batch-1 layer kernels (pi_fast.hip).
//
// A 64-id tile of the predictor's output layer is one workgroup of 8 waves.
// Its phases are written once here: the output layer over the rows of
// positive hidden units (P2 stored hidden-major), FC1 of the tile's active
// GPU-resident neurons against x staged in LDS, and the tile's list segments.
#pragma once
#include "pi_device.h"
#include "pi_b1.h"

namespace pi {

constexpr int kTileIds = 64;                       // neuron ids per output-layer tile (one activation word)
constexpr int kTileWaves = 8;                      // waves per tile workgroup
constexpr int kTileThreads = kTileWaves * kWave;
constexpr int kTileLoads = 16;                     // output-layer row loads in flight per lane (fp16 / fp32)

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave)); }

// The 16-byte vectors one lane reads from one row (issued together), widened and
// dotted later.  Vector u of the lane is row vector u*64 + lane.
template <int DT, int NV>
struct LaneRow {
  uint4 w[NV];
  float sc[NV];
  // rp: the row (wave-uniform; NULL = an absent row, which reads zeros), nvec
  // 16-byte vectors long; sp: its int4 scales.  Lane vectors past the row end
  // read zeros from the buffer range check: no clamped addresses, no branches,
  // and nothing waits on these loads before the dot product.
  __device__ __forceinline__ void issue(const char* rp, const uint16_t* sp, int nvec, int lane) {
    const rsrc_t r = make_rsrc(uniform_ptr(rp), rp ? (uint32_t)nvec * 16u : 0u);
#pragma unroll
    for (int u = 0; u < NV; ++u) w[u] = bload16(r, (uint32_t)(u * kWave + lane) * 16u);
    if constexpr (DT == 2) {
      const rsrc_t rs = make_rsrc(uniform_ptr(sp), sp ? (uint32_t)(nvec / 4) * 2u : 0u);
#pragma unroll
      for (int u = 0; u < NV; ++u) sc[u] = h2f(bload2(rs, (uint32_t)((u * kWave + lane) / 4) * 2u));
    }
    // keep every load of the row ahead of the code that consumes them
    __builtin_amdgcn_sched_barrier(0);
  }
  // Dot product with the lane's x slice held in registers (xr[u] = x[E*v .. E*v+E-1]).
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

// x staged in LDS as E/4 planes of float4: plane p, index v holds
// x[E*v + 4p .. E*v + 4p + 3] (E = elements per 16-byte weight vector), so
// that lane-consecutive vectors read lane-consecutive LDS words.
__host__ __device__ inline int x_npad(int dt, int64_t d) {
  const int nvec = (int)(row_bytes(dt, d) / 16);
  return (nvec + kWave - 1) & ~(kWave - 1);
}
__host__ __device__ inline size_t x_planes_bytes(int dt, int64_t d) {
  return (size_t)(dt == 0 ? 1 : dt == 1 ? 2 : 8) * (size_t)x_npad(dt, d) * 16;
}
// Loads of the staging issued first (registers), written to LDS later, so that
// other loads can be issued in between.  NT threads, rows of NV*64 vectors at most.
template <int DT, int NV, int NT>
struct XStage {
  static constexpr int P = Fmt<DT>::E / 4;
  static constexpr int XQ = (NV * kWave * P + NT - 1) / NT;
  float4v q[XQ];
  __device__ __forceinline__ void load(const float* x, int d) {
    const int nq = d / 4;
    const float4v* x4 = reinterpret_cast<const float4v*>(x);
#pragma unroll
    for (int r = 0; r < XQ; ++r) {
      const int k = r * NT + (int)threadIdx.x;
      q[r] = x4[k < nq ? k : 0];
    }
  }
  __device__ __forceinline__ void store(float4v* xs, int d, int npad) const {
    const int nq = d / 4;
#pragma unroll
    for (int r = 0; r < XQ; ++r) {
      const int k = r * NT + (int)threadIdx.x;
      if (k < nq) xs[(k % P) * npad + k / P] = q[r];
    }
  }
};

// Dot product of a lane's row vectors (vector u at v0 + u*64 + lane, valid below
// vend) with x in LDS planes; the lane's partial sum.  x is read vector by vector,
// so only the row's weights stay in registers.
template <int DT, int NV>
__device__ __forceinline__ float lds_dot(const LaneRow<DT, NV>& rw, const float4v* xs, int npad, int v0, int vend,
                                         int lane) {
  constexpr int E = Fmt<DT>::E, P = E / 4;
  float acc = 0.f;
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int v = v0 + u * kWave + lane;
    const bool vin = v < vend;
    const int vc = vin ? v : 0;
    float xv[E];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const float4v t4 = xs[p * npad + vc];
      xv[4 * p] = vin ? t4.x : 0.f; xv[4 * p + 1] = vin ? t4.y : 0.f;
      xv[4 * p + 2] = vin ? t4.z : 0.f; xv[4 * p + 3] = vin ? t4.w : 0.f;
    }
    float wf[E];
    widen<DT>(rw.w[u], DT == 2 ? rw.sc[u] : 1.f, wf);
#pragma unroll
    for (int e = 0; e < E; ++e) acc = fmaf(wf[e], xv[e], acc);
    __builtin_amdgcn_sched_barrier(0);
  }
  return acc;
}

// Position of the r-th (0-based) set bit of x (r < popcount(x)): a popcount
// descent without branches, so that no control flow separates loads that are
// in flight from their uses.
__device__ __forceinline__ int nth_set_bit64(uint64_t x, int r) {
  int base = 0;
#pragma unroll
  for (int half = 32; half >= 1; half >>= 1) {
    const uint64_t lowmask = (1ull << half) - 1ull;
    const int c = __popcll(x & lowmask);
    const bool up = r >= c;
    r = up ? r - c : r;
    x = up ? (x >> half) : x;
    base = up ? base + half : base;
  }
  return base;
}

// Geometry of the output-layer phase of a tile, for P2's dtype.
template <int PDT>
struct P2Geom {
  static constexpr int EP = Fmt<PDT>::E;             // weights per 16-byte vector
  // row loads in flight per lane: int4 rows hold 32 weights per vector, so a quarter of
  // the loads covers the same rows per pass
  static constexpr int U = PDT == 2 ? kTileLoads / 4 : kTileLoads;
  static constexpr int LPR = kTileIds / EP;          // lanes that cover one row slice of the tile
  static constexpr int RPL = kWave / LPR;            // row slices per wave-wide load
  static constexpr int RP = kTileWaves * RPL * U;    // rows per pass
};

// Output layer of tile `tile` (ids i0 .. i0+63) over the rows m with h[m] > 0:
//   z[i] = sum_m h[m] * P2[m, i]       (c2 not added)
// Lane (sub, cl) of wave w reads slice vector cl of rows m = m0 + (i*8 + w)*RPL + sub.
// hload(m0, hv) fills hv[i] with h of those rows (0 past H); a row with h <= 0 is not
// read (it adds nothing to any logit).  The tile's sums land in red[8][64] (one row
// per wave, the block adds them); returns this lane's count of rows read
// (meaningful where cl == 0).
template <int PDT, class HLoad>
__device__ __forceinline__ int p2_tile_partial(const PredFc1Args& a, int tile, int wave, int lane, HLoad&& hload,
                                               float (*red)[kTileIds]) {
  using G = P2Geom<PDT>;
  constexpr int EP = G::EP, U = G::U, LPR = G::LPR, RPL = G::RPL, RP = G::RP;
  const int H = a.H, N = a.N;
  const int sub = lane / LPR, cl = lane % LPR;
  const int64_t prb = row_bytes(PDT, N);
  const int pvec = (int)(prb / 16);
  int colv = tile * LPR + cl;
  colv = colv < pvec ? colv : pvec - 1;            // past the row end: discarded ids
  const int pgroups = N / 128;
  // the whole matrix as one buffer (the host keeps H * row bytes below 2^31)
  const uint32_t pbytes = (uint32_t)(H * prb);
  const rsrc_t rP = make_rsrc(a.P2, pbytes);
  const rsrc_t rS = make_rsrc(PDT == 2 ? (const void*)a.P2s : a.P2, PDT == 2 ? (uint32_t)H * pgroups * 2u : 0u);
  float acc[EP];
#pragma unroll
  for (int e = 0; e < EP; ++e) acc[e] = 0.f;
  int nact = 0;
  float hv[U];
  for (int m0 = 0; m0 < H; m0 += RP) {
    hload(m0, hv);
    uint4 w[U];
    float sc[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int m = m0 + (i * kTileWaves + wave) * RPL + sub;
      const bool ok = hv[i] > 0.f;               // rows past H read h = 0
      nact += ok ? 1 : 0;
      // a row with h <= 0 gets an offset past the buffer: zeros, no memory request
      w[i] = bload16(rP, ok ? (uint32_t)m * (uint32_t)prb + (uint32_t)colv * 16u : pbytes);
      if constexpr (PDT == 2) sc[i] = h2f(bload2(rS, ok ? (uint32_t)(m * pgroups + colv / 4) * 2u : 0xFFFFFFF0u));
      else sc[i] = 1.f;
    }
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const float hs = hv[i] > 0.f ? hv[i] : 0.f;
      if constexpr (PDT == 2) {
        // int4: the group scale folds into h once per row, and each weight is one
        // signed bit-field extract, one convert and one fma
        const float hsc = hs * sc[i];
        const uint32_t wq[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
          for (int n = 0; n < 8; ++n)
            acc[k * 8 + n] = fmaf((float)((int32_t)(wq[k] << (28 - 4 * n)) >> 28), hsc, acc[k * 8 + n]);
      } else {
        float wf[EP];
        widen<PDT>(w[i], 1.f, wf);
#pragma unroll
        for (int e = 0; e < EP; ++e) acc[e] = fmaf(wf[e], hs, acc[e]);
      }
    }
  }
  // the RPL row groups of the wave hold partial sums of the same ids: butterfly
  // sum (every lane ends with the same bits)
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1)
#pragma unroll
    for (int e = 0; e < EP; ++e) acc[e] += __shfl_xor(acc[e], off, kWave);
  if (sub == 0)
#pragma unroll
    for (int e = 0; e < EP; ++e) red[wave][cl * EP + e] = acc[e];
  return cl == 0 ? nact : 0;
}

// FC1 of a tile's active GPU-resident neurons, row r by wave r % 8 (act = the
// tile's activation word AND the table bitmap Gb; slot = the group prefix gp plus
// the GPU-resident ids below it in the group):
//   a = max(0, W1[slot].x + b1[slot])  (* Wup[slot].x when GATED)
// x is in LDS planes.  Row r's slot and output land in s_slot[r], s_a[r].
template <int DT, int NV, bool GATED, int BDT>
__device__ __forceinline__ void fc1_tile_rows(const PredFc1Args& a, uint64_t act, uint64_t Gb, int gp,
                                              const float4v* xs, int npad, int wave, int lane, int* s_slot,
                                              float* s_a) {
  const int R = __popcll(act);
  const int64_t rb = row_bytes(DT, a.d);
  const int nvec = (int)(rb / 16);
  const int groups = a.d / 128;
  const Bias<BDT> b1_at(a.b1, (uint32_t)a.n_g);
  const char* W1 = reinterpret_cast<const char*>(a.W1);
  const char* Wu = reinterpret_cast<const char*>(a.Wu);
  for (int r = wave; r < R; r += kTileWaves) {
    const int sl = gp + __popcll(Gb & ((1ull << nth_set_bit64(act, r)) - 1ull));
    // a table prepared from another T_g cannot index past W1
    const int s = __builtin_amdgcn_readfirstlane(sl < a.n_g ? sl : -1);
    const float bs = b1_at(s >= 0 ? s : 0);
    LaneRow<DT, NV> rw, ru;
    rw.issue(s >= 0 ? W1 + (int64_t)s * rb : nullptr, DT == 2 && s >= 0 ? a.W1s + (int64_t)s * groups : nullptr, nvec,
             lane);
    if constexpr (GATED)
      ru.issue(s >= 0 ? Wu + (int64_t)s * rb : nullptr, DT == 2 && s >= 0 ? a.Wus + (int64_t)s * groups : nullptr,
               nvec, lane);
    float z = wave_sum(lds_dot<DT, NV>(rw, xs, npad, 0, nvec, lane)) + bs;
    z = z > 0.f ? z : 0.f;
    if constexpr (GATED) z *= wave_sum(lds_dot<DT, NV>(ru, xs, npad, 0, nvec, lane));
    if (lane == 0) {
      s_slot[r] = s;
      s_a[r] = s >= 0 ? z : 0.f;
    }
  }
}

// The list segments of 64-id group grp (called by one whole wave): its ascending
// GPU-resident slots, its ascending cold slots, the (slot, a) pairs with a != 0,
// and the count word.  M: the group's activation word.
__device__ __forceinline__ void write_tile_segments(const PredFc1Args& a, int grp, uint64_t M, uint64_t Gb, int gp,
                                                    const int* s_slot, const float* s_a, int lane) {
  const uint64_t act = M & Gb;
  const int k = __popcll(act);
  const bool in = lane < k;
  const int s = in ? s_slot[lane] : 0;
  const float av = in ? s_a[lane] : 0.f;
  const int64_t base = (int64_t)grp * 64;
  const uint64_t lt = (1ull << lane) - 1ull;
  if (in) a.seg_slot[base + lane] = s;
  const bool nz = in && av != 0.f;
  const uint64_t bn = __ballot(nz);
  if (nz) {
    const int p = __popcll(bn & lt);
    a.pos_slot[base + p] = s;
    a.pos_a[base + p] = av;
  }
  const uint64_t ac = M & ~Gb;
  if ((ac >> lane) & 1ull)
    a.seg_cold[base + __popcll(ac & lt)] = (int32_t)(base + lane - (gp + __popcll(Gb & lt)));
  if (lane == 0) a.cnt[grp] = (uint32_t)k | ((uint32_t)__popcll(ac) << 8) | ((uint32_t)__popcll(bn) << 16);
}

}  // namespace pi
