// pi_fast.hip - batch-1 kernels.
//
// Row dots: every lane owns the same column slice of every row (vectors
// v = u*64 + lane), and all 16-byte loads of a row are issued before the first
// FMA.  The list-driven FC1 of pi_sparse_ffn holds its slice of x in
// registers; the batch-1 hidden layer stages x once per four-wave workgroup in
// LDS planes that hold zeros past the row's end (so the dot reads them with no
// clamp or select), and normalises it on the way in for the chaining call.
//
// The predictor's output layer with its weights stored hidden-major (row m =
// hidden unit m's weights to the N outputs): only the rows of hidden units
// whose ReLU output is positive are read, since a zero hidden unit adds
// nothing to any logit.  One block owns a tile of 64 or 128 neuron ids: each
// lane reads h for its rows and then only the row slices of positive hidden
// units (the others are skipped through the buffer range check), a
// reduce-scatter across the wave's row groups and a sum over the waves give
// the tile's logits, and the block decides the tile's activations.  With int4
// rows a tile's slice is a quarter of a cache line, so neighbouring tiles run
// on one die.  In the fused layer the same block then
// runs FC1 for the tile's active GPU-resident neurons (x staged in LDS) and
// writes the tile's list segments, so no block waits for another.
//
// FC2 of the batch-1 layer over those segments (only rows with a non-zero FC1
// output), with the assembly of the ascending lists, writes one partial per
// chunk of groups; the last launch sums the chunks in order with the merge.
//
// int4 rows (32 weights per 16-byte vector) are decoded one 32-bit word of 8
// weights at a time where registers are scarce (FC1 of the fused layer), and
// FC2 gives each lane one word of each row, so that the decode spreads over
// more waves; each weight is (float)q * scale in the same order either way.
#include "../../include/pi.h"
#include "pi_device.h"
#include "pi_b1.h"

namespace pi {
namespace {

constexpr int kT = 256;
constexpr int kWpb = kT / kWave;
constexpr int kSegUnroll = 16;   // W2 rows in flight per wave in the segment FC2

// Column tiles of 64 16-byte vectors over a row of d elements.
// Column tiles of the segment FC2: one 16-byte vector per lane of each row (fp32 / fp16), one
// 32-bit word (8 weights) per lane for int4 rows, whose decode would otherwise leave few waves
// with much work each.
__host__ __device__ inline int seg_tiles(int dt, int64_t d) {
  const int64_t per_lane = dt == 2 ? 4 : 16;
  return (int)((row_bytes(dt, d) / per_lane + kWave - 1) / kWave);
}

// The lane's slice of x (x[E*v .. E*v + E-1] for v = u*64 + lane) into
// registers, through a buffer over x's nvec*E floats: slices past the end
// read zeros, so no select waits on a load.
template <int DT, int NV>
__device__ __forceinline__ void load_xreg(const float* __restrict__ x, int nvec, int lane,
                                          float (&xr)[NV][Fmt<DT>::E]) {
  constexpr int E = Fmt<DT>::E;
  const rsrc_t r = make_rsrc(uniform_ptr(x), (uint32_t)nvec * E * 4u);
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const uint32_t off = (uint32_t)(u * kWave + lane) * (E * 4u);
#pragma unroll
    for (int q = 0; q < E / 4; ++q) {
      const uint4 t = bload16(r, off + 16u * q);
      xr[u][4 * q + 0] = __uint_as_float(t.x); xr[u][4 * q + 1] = __uint_as_float(t.y);
      xr[u][4 * q + 2] = __uint_as_float(t.z); xr[u][4 * q + 3] = __uint_as_float(t.w);
    }
  }
}

// The 16-byte vectors one lane reads from one row (issued together), widened and
// dotted with the lane's x slice later.
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

// h[j] = max(0, W[j].x + bias[j]) at batch 1, rows up to 32 KB (NV 16-byte vectors per lane): one
// row per wave, its whole row's loads in flight, x staged once per four-wave workgroup in LDS planes
// (plane p, index v holds x[E*v + 4p .. +3]), x (from L2) issued before the row (from HBM) so that
// the staging waits only for x.  Lanes past the row end read zero weights and take zero x.  The dot
// runs over the lane's vectors in order, then the wave sum.  With LN, x is first replaced by its layer
// normalisation, and the grid's first workgroup writes the mean, 1/sqrt(var + eps) and the
// normalised row for the kernels after it.
constexpr int kHidLdsWaves = 4;
template <int DT, int NV, int BDT, bool LN>
__global__ __launch_bounds__(kHidLdsWaves * kWave) void k_hidden_lds(const void* __restrict__ W,
                                                                      const uint16_t* __restrict__ Ws, int rows,
                                                                      int cols, const float* __restrict__ x,
                                                                      const void* __restrict__ bias,
                                                                      float* __restrict__ out,
                                                                      float* __restrict__ ln_stats, float ln_eps,
                                                                      float* __restrict__ x_out) {
  constexpr int E = Fmt<DT>::E;
  constexpr int P = E / 4;                                 // x planes
  constexpr int NT = kHidLdsWaves * kWave;
  constexpr int XQ = (NV * kWave * P + NT - 1) / NT;       // x float4 per thread
  extern __shared__ __attribute__((aligned(16))) char hl_smem[];
  float4v* xs = reinterpret_cast<float4v*>(hl_smem);
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = wave_id();
  const int j = blockIdx.x * kHidLdsWaves + wave;
  const bool row_ok = j < rows;
  const int64_t rb = row_bytes(DT, cols);
  const int nvec = (int)(rb / 16);
  const int npad = NV * kWave;                             // plane stride: every u < NV in bounds
  const int nq = cols / 4;
  const float4v* x4 = reinterpret_cast<const float4v*>(x);
  float4v xq[XQ];
#pragma unroll
  for (int r = 0; r < XQ; ++r) {
    const int q = r * NT + tid;
    xq[r] = x4[q < nq ? q : 0];
  }
  const Bias<BDT> bias_at(bias, (uint32_t)rows);
  const float bj = bias_at(row_ok ? j : 0);
  LaneRow<DT, NV> rw;
  rw.issue(row_ok ? reinterpret_cast<const char*>(W) + (int64_t)j * rb : nullptr,
           DT == 2 && row_ok ? Ws + (int64_t)j * (cols / 128) : nullptr, nvec, lane);
  if constexpr (LN) {
    // x replaced by its layer normalisation (unit gain, zero bias): the mean, then the population
    // variance, each summed over the thread's staged values in order, the wave butterfly and the
    // waves in wave order (every workgroup the same partition, so the same two values), while the
    // row is still arriving; x becomes fma(x, inv, -mean * inv), the form the next kernel applies
    // to its own copy with the two values written here
    __shared__ float part[2][kHidLdsWaves];
    float sa = 0.f;
#pragma unroll
    for (int r = 0; r < XQ; ++r)
      if (r * NT + tid < nq) { sa += xq[r].x; sa += xq[r].y; sa += xq[r].z; sa += xq[r].w; }
    sa = wave_sum(sa);
    if (lane == 0) part[0][wave] = sa;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kHidLdsWaves; ++w) tot += part[0][w];
    const float mu = tot / (float)cols;
    float sq = 0.f;
#pragma unroll
    for (int r = 0; r < XQ; ++r)
      if (r * NT + tid < nq) {
        const float d0 = xq[r].x - mu, d1 = xq[r].y - mu, d2 = xq[r].z - mu, d3 = xq[r].w - mu;
        sq += d0 * d0; sq += d1 * d1; sq += d2 * d2; sq += d3 * d3;
      }
    sq = wave_sum(sq);
    if (lane == 0) part[1][wave] = sq;
    __syncthreads();
    float var = 0.f;
#pragma unroll
    for (int w = 0; w < kHidLdsWaves; ++w) var += part[1][w];
    const float inv = 1.0f / sqrtf(var / (float)cols + ln_eps);
    const float nm = -mu * inv;
#pragma unroll
    for (int r = 0; r < XQ; ++r) {
      xq[r].x = fmaf(xq[r].x, inv, nm); xq[r].y = fmaf(xq[r].y, inv, nm);
      xq[r].z = fmaf(xq[r].z, inv, nm); xq[r].w = fmaf(xq[r].w, inv, nm);
    }
    if (blockIdx.x == 0) {               // the grid's first workgroup reports them
      if (x_out) {
#pragma unroll
        for (int r = 0; r < XQ; ++r) {
          const int q = r * NT + tid;
          if (q < nq) reinterpret_cast<float4v*>(x_out)[q] = xq[r];
        }
      }
      if (tid == 0) { ln_stats[0] = mu; ln_stats[1] = inv; }
    }
  }
#pragma unroll
  for (int r = 0; r < XQ; ++r) {
    const int q = r * NT + tid;
    if (q < nq) xs[(q % P) * npad + q / P] = xq[r];
  }
  // the planes past the row's end hold zeros, so the dot reads them unconditionally
  for (int q = nvec + tid; q < npad; q += NT) {
#pragma unroll
    for (int p = 0; p < P; ++p) xs[p * npad + q] = float4v{0.f, 0.f, 0.f, 0.f};
  }
  __syncthreads();
  if (!row_ok) return;
  float acc = 0.f;
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    // past the row's end the weights and x both read zeros: no index clamp, no select
    const int v = u * kWave + lane;
    float xv[E];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const float4v t4 = xs[p * npad + v];
      xv[4 * p] = t4.x; xv[4 * p + 1] = t4.y; xv[4 * p + 2] = t4.z; xv[4 * p + 3] = t4.w;
    }
    float wf[E];
    widen<DT>(rw.w[u], DT == 2 ? rw.sc[u] : 1.f, wf);
#pragma unroll
    for (int e = 0; e < E; ++e) acc = fmaf(wf[e], xv[e], acc);
  }
  float z = wave_sum(acc) + bj;
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
  const int gw = blockIdx.x * kWpb + wave;
  if (gw >= n_g) return;
  const int64_t rb = row_bytes(DT, cols);
  const int nvec = (int)(rb / 16);
  const int groups = cols / 128;
  const Bias<BDT> bias_at(bias, (uint32_t)n_g);
  int K = *Kp;                       // issued with the list entry (no dependency between them)
  int s = __builtin_amdgcn_readfirstlane(list[gw]);
  K = K < 0 ? 0 : (K > n_g ? n_g : K);
  if (gw >= K) return;
  {
    const int j = gw;                // the grid has one wave per possible list entry
    const bool ok = s >= 0 && s < n_g;
    const float bs = bias_at(ok ? s : 0);
    LaneRow<DT, NV> r, u;
    r.issue(ok ? reinterpret_cast<const char*>(W) + (int64_t)s * rb : nullptr,
            DT == 2 && ok ? Ws + (int64_t)s * groups : nullptr, nvec, lane);
    if constexpr (GATED)
      u.issue(ok ? reinterpret_cast<const char*>(Wu) + (int64_t)s * rb : nullptr,
              DT == 2 && ok ? Wus + (int64_t)s * groups : nullptr, nvec, lane);
    float xr[NV][Fmt<DT>::E];
    load_xreg<DT, NV>(x, nvec, lane, xr);
    __builtin_amdgcn_sched_barrier(0);   // all of x in flight before the first FMA
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
    const uint64_t lowmask = (1ull << half) - 1ull;
    const int c = __popcll(x & lowmask);
    const bool up = r >= c;
    r = up ? r - c : r;
    x = up ? (x >> half) : x;
    base = up ? base + half : base;
  }
  return base;
}

// Workgroups go to the eight dies round robin by index, and each die has its own L2.  Tile t of
// the first (n / 8) * 8 runs on die t / (n / 8): neighbouring tiles share a die, so a cache line
// that holds several tiles' slices (an int4 P2 row: 32 bytes per 64-id tile) is fetched into one L2.
__device__ __forceinline__ int xcd_tile(int b, int n) {
  constexpr int kDies = 8;
  const int per = n / kDies;
  if (b >= per * kDies) return b;
  return (b % kDies) * per + b / kDies;
}

// Geometry of the output-layer tile kernel for T neuron ids per block.
template <int T>
struct TileGeom {
  static constexpr int W = T / 8;                    // waves: 8 for 64 ids, 16 for 128 ids
  static constexpr int NT = W * kWave;
  static constexpr int NG = T / 64;                  // 64-id groups per tile
  static constexpr int U = 16;                       // row loads in flight per lane (T=128: 1024 rows per pass)
};

__host__ __device__ constexpr size_t align16(size_t v) { return (v + 15) & ~(size_t)15; }


// Output layer (+ FC1) of one tile of T neuron ids [i0, i0 + T):
//   z_i = c2_i + sum over hidden units m with h_m > 0 of h_m * P2[m, i]
//   activation bit_i = z_i > tau   (ids >= N inactive)
// and with FC1, for the tile's active GPU-resident neurons (activation AND the
// prepared table's bitmap; slot = the table prefix of the 64-id group plus the
// GPU-resident ids below it in the group):
//   a = max(0, W1[slot].x + b1[slot]) (* Wup[slot].x when GATED)
// Each 64-id group of the tile receives its ascending slot segment, its
// ascending cold-slot segment, the (slot, a) pairs with a != 0 (the only FC2
// rows that contribute) and the three counts.
template <int PDT, int DT, int NV, bool GATED, int BDT, int T, bool FC1>
__global__ __launch_bounds__(T * 8) void k_pred_fc1(PredFc1Args a) {
  using G = TileGeom<T>;
  constexpr int EP = Fmt<PDT>::E;      // output-layer weights per 16-byte vector
  // row loads in flight per lane: int4 rows hold 32 weights per vector, so a quarter of
  // the loads covers the same rows per pass (and keeps two blocks per compute unit)
  constexpr int W = G::W, NT = G::NT, NG = G::NG, U = PDT == 2 ? G::U / 4 : G::U;
  constexpr int LPR = T / EP;          // lanes that cover one row slice of the tile
  constexpr int RPL = kWave / LPR;     // row slices per wave-wide load
  constexpr int E = Fmt<DT>::E;        // FC1 weights per 16-byte vector
  constexpr int P = E / 4;             // x planes
  constexpr int XQ = (NV * kWave * P + NT - 1) / NT;   // x float4 per thread
  extern __shared__ __attribute__((aligned(16))) char pf_smem[];
  __shared__ float red[W][T];
  __shared__ float s_a[T];
  __shared__ int s_slot[T];

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = wave_id();
  const int H = a.H, N = a.N;
  const int ngroups = (N + 63) / 64;
  const int ntl = (N + T - 1) / T;
  // int4 P2 rows give each tile a 32-byte slice: its neighbours share the line, so they share a die
  const int tile = PDT == 2 && (int)blockIdx.x < ntl ? xcd_tile((int)blockIdx.x, ntl) : (int)blockIdx.x;
  const int64_t i0 = (int64_t)tile * T;
  float4v* xs = reinterpret_cast<float4v*>(pf_smem);

  // ---- issue: table words, bias, x, h
  uint64_t Gb[NG];
  int gp[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int grp = tile * NG + g;
    const bool in = FC1 && grp < ngroups;
    Gb[g] = in ? ((uint64_t)a.gbits[2 * grp] | ((uint64_t)a.gbits[2 * grp + 1] << 32)) : 0ull;
    gp[g] = in ? a.gpre[grp] : 0;
  }
  // every wave takes the tile's activation decision itself (the same sums in the same order, so
  // the same bits in every wave): c2 of the lane's id in each 64-id group
  const Bias<BDT> c2_at(a.c2, (uint32_t)N);
  float c2v[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int64_t idg = i0 + g * kWave + lane;
    c2v[g] = c2_at(idg < N ? idg : 0);
  }
  const int nvec = FC1 ? (int)(row_bytes(DT, a.d) / 16) : 0;
  const int npad = FC1 ? NV * kWave : 0;                  // plane stride: every u < NV in bounds
  float4v xq[FC1 ? XQ : 1];
  // x given raw with the statistics the hidden-layer kernel left: normalised on the way into LDS
  // with the same two values and the same fma, so FC1 sees the hidden layer's x bit for bit
  float ln_inv = 1.f, ln_nm = 0.f;
  if (FC1 && a.ln_stats) { ln_inv = a.ln_stats[1]; ln_nm = -a.ln_stats[0] * ln_inv; }
  if constexpr (FC1) {
    const int nq = a.d / 4;
    const float4v* x4 = reinterpret_cast<const float4v*>(a.x);
#pragma unroll
    for (int r = 0; r < XQ; ++r) {
      const int q = r * NT + tid;
      xq[r] = x4[q < nq ? q : 0];
    }
  }
  // lane (sub, cl) reads slice vector cl of rows m = (i*W + wave)*RPL + sub of each
  // pass of RP rows, and first its h[m]: rows with h[m] <= 0 get an offset past
  // the buffer, which reads zeros without a memory request (no compaction, no
  // barrier before the weight loads)
  constexpr int RP = W * RPL * U;
  const int sub = lane / LPR, cl = lane % LPR;
  const rsrc_t rH = make_rsrc(a.h, (uint32_t)H * 4u);
  float hv[U];
#pragma unroll
  for (int i = 0; i < U; ++i)
    hv[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rH, ((i * W + wave) * RPL + sub) * 4, 0, 0));
  if constexpr (FC1) {
    // x in planes: plane p, index v holds x[E*v + 4p .. +3]
    const int nq = a.d / 4;
#pragma unroll
    for (int r = 0; r < XQ; ++r) {
      const int q = r * NT + tid;
      if (q < nq) {
        float4v v = xq[r];
        if (a.ln_stats) {
          v.x = fmaf(v.x, ln_inv, ln_nm); v.y = fmaf(v.y, ln_inv, ln_nm);
          v.z = fmaf(v.z, ln_inv, ln_nm); v.w = fmaf(v.w, ln_inv, ln_nm);
        }
        xs[(q % P) * npad + q / P] = v;
      }
    }
    // the planes past the row's end hold zeros, so the row dots read them unconditionally
    for (int q = nvec + tid; q < npad; q += NT) {
#pragma unroll
      for (int p = 0; p < P; ++p) xs[p * npad + q] = float4v{0.f, 0.f, 0.f, 0.f};
    }
  }

  if constexpr (FC1) {
    // ---- look-ahead blocks: one row of the next layer's predictor hidden layer per wave, on
    // the x this block has staged (block-uniform branch)
    const int ntiles = (N + T - 1) / T;
    if (a.nh && (int)blockIdx.x >= ntiles) {
      __syncthreads();
      const int m = ((int)blockIdx.x - ntiles) * W + wave;
      if (m < a.nH) {
        const int64_t rb = row_bytes(DT, a.d);
        const int groups = a.d / 128;
        const Bias<BDT> c1_at(a.nc1, (uint32_t)a.nH);
        LaneRow<DT, NV> rw;
        rw.issue(reinterpret_cast<const char*>(a.nP1) + (int64_t)m * rb, DT == 2 ? a.nP1s + (int64_t)m * groups : nullptr,
                 nvec, lane);
        float a0 = 0.f;
#pragma unroll
        for (int u = 0; u < NV; ++u) {
          const int v = u * kWave + lane;    // past the row's end: zero weights and zero x
          float xv[E];
#pragma unroll
          for (int p = 0; p < P; ++p) {
            const float4v t4 = xs[p * npad + v];
            xv[4 * p] = t4.x; xv[4 * p + 1] = t4.y; xv[4 * p + 2] = t4.z; xv[4 * p + 3] = t4.w;
          }
          float wf[E];
          widen<DT>(rw.w[u], DT == 2 ? rw.sc[u] : 1.f, wf);
#pragma unroll
          for (int e = 0; e < E; ++e) a0 = fmaf(wf[e], xv[e], a0);
          __builtin_amdgcn_sched_barrier(0);
        }
        float z = wave_sum(a0) + c1_at(m);
        z = z > 0.f ? z : 0.f;
        if (lane == 0) a.nh[m] = z;
      }
      return;
    }
  }

  // ---- output layer over the rows of positive hidden units
  {
    const int64_t prb = row_bytes(PDT, N);
    const int pvec = (int)(prb / 16);
    int colv = tile * LPR + cl;
    colv = colv < pvec ? colv : pvec - 1;          // past the row end: discarded ids
    const int pgroups = N / 128;
    // the whole matrix as one buffer (the host keeps H * row bytes below 2^31)
    const uint32_t pbytes = (uint32_t)(H * prb);
    const rsrc_t rP = make_rsrc(a.P2, pbytes);
    const rsrc_t rS = make_rsrc(PDT == 2 ? (const void*)a.P2s : a.P2, PDT == 2 ? (uint32_t)H * pgroups * 2u : 0u);
    float acc[EP];
#pragma unroll
    for (int e = 0; e < EP; ++e) acc[e] = 0.f;
    for (int m0 = 0; m0 < H; m0 += RP) {
      if (m0 > 0) {
#pragma unroll
        for (int i = 0; i < U; ++i)
          hv[i] = __uint_as_float(
              __builtin_amdgcn_raw_buffer_load_b32(rH, (m0 + (i * W + wave) * RPL + sub) * 4, 0, 0));
      }
      uint4 w[U];
      float sc[U];
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const int m = m0 + (i * W + wave) * RPL + sub;
        const bool ok = hv[i] > 0.f;               // rows past H read h = 0
        w[i] = bload16(rP, ok ? (uint32_t)m * (uint32_t)prb + (uint32_t)colv * 16u : pbytes);
        if constexpr (PDT == 2) sc[i] = h2f(bload2(rS, ok ? (uint32_t)(m * pgroups + colv / 4) * 2u : 0xFFFFFFF0u));
        else sc[i] = 1.f;
      }
#pragma unroll
      for (int i = 0; i < U; ++i) {
        // h is a ReLU output (>= +0), and a row not read has zero weights: h needs no select
        const float hs = hv[i];
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
    // the RPL row groups of the wave hold partial sums of the same ids: a reduce-scatter over
    // them, whose pairwise sums are a butterfly's (partner groups sub and sub ^ 2^s, s ascending),
    // each computed once, in the lane that keeps that id.  At step s a lane holds n = EP >> s ids
    // and keeps the half that bit s of sub selects, so lane (cl, sub) ends with EP / RPL ids'
    // sums: log2(RPL) steps of n / 2 exchanges (31 for int4 rows, against 160 for every lane
    // summing all EP ids), the same bits.
    static_assert(EP % RPL == 0 && (RPL & (RPL - 1)) == 0, "row groups: a power of two dividing EP");
    int base = 0;
#pragma unroll
    for (int st = 0; (LPR << st) < kWave; ++st) {
      const int h = (EP >> st) / 2;
      const bool up = ((sub >> st) & 1) != 0;
#pragma unroll
      for (int i = 0; i < h; ++i) {
        const float keep = up ? acc[h + i] : acc[i];
        const float give = up ? acc[i] : acc[h + i];
        acc[i] = keep + __shfl_xor(give, LPR << st, kWave);
      }
      base += up ? h : 0;
    }
#pragma unroll
    for (int i = 0; i < EP / RPL; ++i) red[wave][cl * EP + base + i] = acc[i];
  }
  if (a.rows_read && tile == 0 && wave == 0) {   // the P2 rows read: hidden units with h > 0
    int c = 0;
    for (int m = lane; m < H; m += kWave) c += a.h[m] > 0.f ? 1 : 0;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off, kWave);
    if (lane == 0) *a.rows_read = c;
  }
  __syncthreads();
  uint64_t Mb[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int c = g * kWave + lane;
    float z = red[0][c];
#pragma unroll
    for (int w2 = 1; w2 < W; ++w2) z += red[w2][c];
    z += c2v[g];
    const int64_t idg = i0 + c;
    const bool valid = idg < N;
    Mb[g] = __ballot(valid && z > a.tau);
    if (wave == g) {                  // wave g reports group g
      if (a.logits && valid) a.logits[idg] = z;
      const int grp = tile * NG + g;
      if (!FC1 && a.mask && lane == 0 && grp < ngroups) {
        a.mask[2 * grp] = (uint32_t)Mb[g];
        a.mask[2 * grp + 1] = (uint32_t)(Mb[g] >> 32);
      }
    }
  }
  if constexpr (!FC1) return;

  // ---- FC1 of the tile's active GPU-resident neurons, row r by wave r % W
  uint64_t act[NG];
  int kg[NG];
  int R = 0;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    act[g] = Mb[g] & Gb[g];
    kg[g] = __popcll(act[g]);
    R += kg[g];
  }
  {
    const int64_t rb = row_bytes(DT, a.d);
    const int groups = a.d / 128;
    const Bias<BDT> b1_at(a.b1, (uint32_t)a.n_g);
    const char* W1 = reinterpret_cast<const char*>(a.W1);
    const char* Wu = reinterpret_cast<const char*>(a.Wu);
    for (int r = wave; r < R; r += W) {
      const int g = (NG == 2 && r >= kg[0]) ? 1 : 0;
      const int t = g ? r - kg[0] : r;
      const int sl = gp[g] + __popcll(Gb[g] & ((1ull << nth_set_bit64(act[g], t)) - 1ull));
      // a table prepared from another T_g cannot index past W1
      const int s = __builtin_amdgcn_readfirstlane(sl < a.n_g ? sl : -1);
      const float bs = b1_at(s >= 0 ? s : 0);
      LaneRow<DT, NV> rw, ru;
      rw.issue(s >= 0 ? W1 + (int64_t)s * rb : nullptr, DT == 2 && s >= 0 ? a.W1s + (int64_t)s * groups : nullptr,
               nvec, lane);
      if constexpr (GATED)
        ru.issue(s >= 0 ? Wu + (int64_t)s * rb : nullptr, DT == 2 && s >= 0 ? a.Wus + (int64_t)s * groups : nullptr,
                 nvec, lane);
      float a0 = 0.f, g0 = 0.f;
      if constexpr (DT == 2) {
        // int4: one 32-bit word (8 weights, x planes 2i and 2i+1) at a time, the next word's x read
        // from LDS before this word is decoded; each weight is (float)q * scale as widen gives it,
        // in the same order, so the bits are widen's
        auto xword = [&](int u, int i, float (&xo)[8]) {
          const int v = u * kWave + lane;    // past the row's end: zero weights and zero x
          const float4v t0 = xs[(2 * i) * npad + v], t1 = xs[(2 * i + 1) * npad + v];
          xo[0] = t0.x; xo[1] = t0.y; xo[2] = t0.z; xo[3] = t0.w;
          xo[4] = t1.x; xo[5] = t1.y; xo[6] = t1.z; xo[7] = t1.w;
        };
        auto word = [](const uint4& w, int i) { return i == 0 ? w.x : i == 1 ? w.y : i == 2 ? w.z : w.w; };
        float xa[8], xb[8];
        xword(0, 0, xa);
#pragma unroll
        for (int c = 0; c < 4 * NV; ++c) {
          const int u = c / 4, i = c % 4;
          if (c + 1 < 4 * NV) xword((c + 1) / 4, (c + 1) % 4, xb);
          const uint32_t wa = word(rw.w[u], i);
#pragma unroll
          for (int n = 0; n < 8; ++n) {
            int q = (int)((wa >> (4 * n)) & 0xF);
            q = (q ^ 8) - 8;
            a0 = fmaf((float)q * rw.sc[u], xa[n], a0);
          }
          if constexpr (GATED) {
            const uint32_t wg = word(ru.w[u], i);
#pragma unroll
            for (int n = 0; n < 8; ++n) {
              int q = (int)((wg >> (4 * n)) & 0xF);
              q = (q ^ 8) - 8;
              g0 = fmaf((float)q * ru.sc[u], xa[n], g0);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int n = 0; n < 8; ++n) xa[n] = xb[n];
        }
      } else {
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const int v = u * kWave + lane;      // past the row's end: zero weights and zero x
        float xv[E];
#pragma unroll
        for (int p = 0; p < P; ++p) {
          const float4v t4 = xs[p * npad + v];
          xv[4 * p] = t4.x; xv[4 * p + 1] = t4.y; xv[4 * p + 2] = t4.z; xv[4 * p + 3] = t4.w;
        }
        float wf[E];
        widen<DT>(rw.w[u], DT == 2 ? rw.sc[u] : 1.f, wf);
#pragma unroll
        for (int e = 0; e < E; ++e) a0 = fmaf(wf[e], xv[e], a0);
        if constexpr (GATED) {
          widen<DT>(ru.w[u], DT == 2 ? ru.sc[u] : 1.f, wf);
#pragma unroll
          for (int e = 0; e < E; ++e) g0 = fmaf(wf[e], xv[e], g0);
        }
        // x is read from LDS vector by vector: keeps only the row's weights in
        // registers (other waves cover the LDS latency)
        __builtin_amdgcn_sched_barrier(0);
      }
      }
      float z = wave_sum(a0) + bs;
      z = z > 0.f ? z : 0.f;
      if constexpr (GATED) z *= wave_sum(g0);
      if (lane == 0) {
        s_slot[r] = s;
        s_a[r] = s >= 0 ? z : 0.f;
      }
    }
  }
  __syncthreads();

  // ---- segments of each 64-id group, by wave g
  if (wave < NG) {
    const int g = wave;
    const int grp = tile * NG + g;
    if (grp < ngroups) {
      const int r0 = g == 0 ? 0 : kg[0];
      const int k = kg[g];
      const bool in = lane < k;
      const int s = in ? s_slot[r0 + lane] : 0;
      const float av = in ? s_a[r0 + lane] : 0.f;
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
      const uint64_t ac = Mb[g] & ~Gb[g];
      if ((ac >> lane) & 1ull)
        a.seg_cold[base + __popcll(ac & lt)] = (int32_t)(base + lane - (gp[g] + __popcll(Gb[g] & lt)));
      if (lane == 0) a.cnt[grp] = (uint32_t)k | ((uint32_t)__popcll(ac) << 8) | ((uint32_t)__popcll(bn) << 16);
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

// Vectors per lane of the fused kernel's FC1 rows, whose x is in LDS (not registers): the row's
// loads alone bound it, 16 vectors for fp32 / fp16 rows and 8 for int4 rows (32 weights each).
// The steps of 10, 12 and 14 keep a gated layer's two rows (W1 and Wup, both in flight) to the
// registers they need (at d = 5,120 fp16, 121 VGPRs, four waves per SIMD, against 187, two), and
// every row's dot to the vectors it has (14 at d = 7,168 fp16: a vector past the row's end still
// costs its LDS reads and fmas).
template <int DT>
int pick_nv_fused(int nvec) {
  for (int nv : {4, 8, 10, 12, 14, 16}) {
    if (DT == 2 && nv > 8) break;
    if (nv * kWave >= nvec) return nv;
  }
  return 0;
}

int pick_nv_rt(int dt, int nvec) {
  switch (dt) {
    case 0: return pick_nv<0>(nvec);
    case 1: return pick_nv<1>(nvec);
    default: return pick_nv<2>(nvec);
  }
}

int grid_for(int64_t waves, int cap) {
  int64_t b = (waves + kWpb - 1) / kWpb;
  return (int)(b < 1 ? 1 : (b > cap ? cap : b));
}

// Vectors per lane of k_hidden_lds for a row of nvec 16-byte vectors (0 = unsupported): 8, 10, 12,
// 14, 16, 24 or 32 (int4: 4, 8 or 16, whose x takes a quarter of the registers per vector).  A
// vector past the row's end still costs registers and its share of the dot, so the steps follow
// the common widths: 10 at d = 5,120 and 14 at d = 7,168 fp16, 4 for the 3.5 KB int4 rows at
// d = 7,168 (123 VGPRs at 8, 64 of them for x on its way to LDS).
template <int DT>
int pick_nv_lds(int nvec) {
  for (int nv : {4, 8, 10, 12, 14, 16, 24, 32}) {
    if (DT != 2 && nv < 8) continue;
    if (DT == 2 && nv > 8 && nv < 16) continue;
    if (DT == 2 && nv > 16) break;
    if (nv * kWave >= nvec) return nv;
  }
  return 0;
}

template <int DT>
hipError_t hidden_lds_dt(const B1Gemv& g, hipStream_t s) {
  const int nvec = (int)(row_bytes(DT, g.cols) / 16);
  const size_t shm = (size_t)pick_nv_lds<DT>(nvec) * kWave * (Fmt<DT>::E / 4) * 16;   // planes of NV * 64
  const dim3 gr((unsigned)((g.rows + kHidLdsWaves - 1) / kHidLdsWaves)), bl(kHidLdsWaves * kWave);
#define PI_HL_LN(NVV, BB)                                                                                   \
  do {                                                                                                      \
    if (g.ln_stats)                                                                                         \
      hipLaunchKernelGGL((k_hidden_lds<DT, NVV, BB, true>), gr, bl, shm, s, g.W, g.Ws, g.rows, g.cols, g.x,   \
                         g.bias, g.out, g.ln_stats, g.ln_eps, g.x_out);                                     \
    else                                                                                                    \
      hipLaunchKernelGGL((k_hidden_lds<DT, NVV, BB, false>), gr, bl, shm, s, g.W, g.Ws, g.rows, g.cols, g.x,  \
                         g.bias, g.out, nullptr, 0.f, nullptr);                                             \
  } while (0)
#define PI_HL(NVV)                                                                                          \
  do {                                                                                                      \
    if (g.bias && g.bias_dt == 0) PI_HL_LN(NVV, 0);                                                         \
    else PI_HL_LN(NVV, 1);                                                                                  \
  } while (0)
  switch (pick_nv_lds<DT>(nvec)) {
    case 4: if constexpr (DT == 2) PI_HL(4); break;
    case 8: PI_HL(8); break;
    case 10: if constexpr (DT != 2) PI_HL(10); break;
    case 12: if constexpr (DT != 2) PI_HL(12); break;
    case 14: if constexpr (DT != 2) PI_HL(14); break;
    case 16: PI_HL(16); break;
    case 24: if constexpr (DT != 2) PI_HL(24); break;
    case 32: if constexpr (DT != 2) PI_HL(32); break;
    default: return hipErrorInvalidValue;
  }
#undef PI_HL
#undef PI_HL_LN
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

// Tile width: 64 ids per block of 8 waves.  (128-id tiles of 16 waves measured
// slower at the OPT-30B shape: two co-resident 64-id blocks per CU hide each
// other's barrier waits.)
constexpr int kTile = 64;

template <int PDT, int DT, int NV, bool GATED, int BDT, int T, bool FC1>
hipError_t pf_launch(const PredFc1Args& a, hipStream_t s) {
  unsigned blocks = (unsigned)((a.N + T - 1) / T);
  if (FC1 && a.nh) blocks += (unsigned)((a.nH + 7) / 8);   // look-ahead rows, T / 8 = 8 waves per block
  size_t shm = 0;                     // x in E/4 planes of float4 when FC1 runs
  if constexpr (FC1) shm += (size_t)(Fmt<DT>::E / 4) * NV * kWave * 16;   // planes of NV * 64 vectors
  hipLaunchKernelGGL((k_pred_fc1<PDT, DT, NV, GATED, BDT, T, FC1>), dim3(blocks), dim3(T * 8), shm, s, a);
  return hipGetLastError();
}

template <int PDT, int BDT>
hipError_t pred_out_pdt(const PredFc1Args& a, hipStream_t s) {
  return pf_launch<PDT, 0, 1, false, BDT, kTile, false>(a, s);
}

// Fused kernels exist for these (output-layer dtype, FFN dtype, bias dtype)
// combinations: all fp32, fp16 predictor + fp16 FFN, fp16 predictor + int4 FFN,
// int4 predictor + fp16 FFN (fp16 biases); fp32 gated layers take the separate
// kernels.
template <int PDT, int DT, int BDT, bool GATED>
hipError_t pred_fc1_combo(const PredFc1Args& a, hipStream_t s) {
  const int nv = pick_nv_fused<DT>((int)(row_bytes(DT, a.d) / 16));
#define PI_PF(NVV) return pf_launch<PDT, DT, NVV, GATED, BDT, kTile, true>(a, s)
  switch (nv) {
    case 4: PI_PF(4);
    case 8: PI_PF(8);
    case 10: if constexpr (Fmt<DT>::E <= 8) PI_PF(10);
    case 12: if constexpr (Fmt<DT>::E <= 8) PI_PF(12);
    case 14: if constexpr (Fmt<DT>::E <= 8) PI_PF(14);
    case 16: if constexpr (Fmt<DT>::E <= 8) PI_PF(16);
    default: return hipErrorInvalidValue;
  }
#undef PI_PF
}

// Batch-1 FC2 over the group segments of the fused layer, and the list
// assembly.  Blocks [0, tiles * kSegChunks) are FC2 blocks: block (tile,
// chunk) takes the groups [c * ngroups / C, (c + 1) * ngroups / C); its rows are
// those groups' (slot, a) pairs with a != 0 in group order (ascending slots),
// gathered into LDS first (one round trip), then the listed W2 rows are
// streamed over the block's column tile: 16-byte loads (a 32-bit word for int4), kSegUnroll rows in
// flight per wave.  It writes one partial per chunk.  The other blocks each
// place 256 entries (four groups) of the ascending lists A_g / A_c, at offsets
// from the counts of the groups below; list block 0 writes K and K_c.
template <int DT>
__global__ __launch_bounds__(kT) void k_fc2_seg(Fc2SegArgs a, int tiles) {
  constexpr int E = DT == 2 ? 8 : Fmt<DT>::E;   // columns per lane (int4: one 32-bit word)
  extern __shared__ int32_t fsm[];
  __shared__ float red[kWpb][kWave * E];
  __shared__ int s_cnt[64];
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
  // the group counts first, then each thread's share of the raw (slot, a) entries: wave w takes
  // the entries of groups w, w + 4, ... (lane = entry in the group), so every group is one wave's.
  // Each wave scans the counts itself (the same offsets in every wave), so the compaction needs
  // one barrier, after the entries are placed.
  constexpr int RQ = 16;   // groups per wave: nb <= RQ * kWpb
  const int cv = lane < nb ? (int)cnt_nz(a.cnt[b0 + lane]) : 0;
  int32_t rs[RQ];
  float ra[RQ];
#pragma unroll
  for (int q = 0; q < RQ; ++q) {
    const int e = q * kT + tid;
    rs[q] = e < nb * 64 ? a.pos_slot[(int64_t)b0 * 64 + e] : -1;
    ra[q] = e < nb * 64 ? a.pos_a[(int64_t)b0 * 64 + e] : 0.f;
  }
  int incl = cv;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int t = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += t;
  }
  const int excl = incl - cv;
  const int R = __builtin_amdgcn_readlane(incl, kWave - 1);
#pragma unroll
  for (int q = 0; q < RQ; ++q) {
    const int bb = q * kWpb + wave;          // this wave's group at step q (wave-uniform)
    if (bb < nb) {
      const int cb = __builtin_amdgcn_readlane(cv, bb), ob = __builtin_amdgcn_readlane(excl, bb);
      if (lane < cb) {
        c_slot[ob + lane] = rs[q];
        c_a[ob + lane] = ra[q];
      }
    }
  }
  __syncthreads();
  const int64_t d = a.d;
  const int64_t rb = row_bytes(DT, d);
  // the lane's unit of each row: a 16-byte vector, or for int4 a 32-bit word (8 weights)
  constexpr int UB = DT == 2 ? 4 : 16;
  const int nunit = (int)(rb / UB);
  const int v = tile * kWave + lane;
  const bool vok = v < nunit;
  const int64_t groups = d / 128;
  const int64_t tile_col0 = (int64_t)tile * kWave * E;
  const char* W2 = reinterpret_cast<const char*>(a.W2);
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int jb = wave; jb < R; jb += kWpb * kSegUnroll) {
    uint4 w[DT == 2 ? 1 : kSegUnroll];
    uint32_t wq[DT == 2 ? kSegUnroll : 1];
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
      if constexpr (DT == 2) {
        wq[u] = __builtin_amdgcn_raw_buffer_load_b32(rw, (int)(v * UB), 0, 0);
        const rsrc_t rs = make_rsrc(a.W2s + (s >= 0 ? (int64_t)s * groups : 0), s >= 0 ? (uint32_t)groups * 2u : 0u);
        scl[u] = h2f(bload2(rs, (uint32_t)(v / 16) * 2u));   // 16 words per 128-weight group
      } else {
        w[u] = bload16(rw, (uint32_t)v * 16u);
      }
    }
#pragma unroll
    for (int u = 0; u < kSegUnroll; ++u) {
      if constexpr (DT == 2) {
        // each weight is (float)q * scale, as widen gives it
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          int q = (int)((wq[u] >> (4 * n)) & 0xF);
          q = (q ^ 8) - 8;
          acc[n] = fmaf(ab[u], (float)q * scl[u], acc[n]);
        }
      } else {
        float wf[E];
        widen<DT>(w[u], 1.f, wf);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = fmaf(ab[u], wf[e], acc[e]);
      }
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
  // the partials through one buffer: the column's byte offset per lane and each chunk's as a
  // scalar, so the 32 loads go out with no address arithmetic between them
  const rsrc_t rp = make_rsrc(r.partials, (uint32_t)(kSegChunks * r.d * 4));
  float p[kSegChunks];
#pragma unroll
  for (int c = 0; c < kSegChunks; ++c)
    p[c] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rp, (int)(t * 4), (int)(c * r.d * 4), 0));
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < kSegChunks; ++c) sum += p[c];
  if (r.y_c && kc != 0) sum += yc;
  if (r.b2) sum += bb;
  r.y[t] = sum;
}
}  // namespace

bool b1_supported(int dt, int64_t cols) {
  const int nvec = (int)(row_bytes(dt, cols) / 16);
  return pick_nv_rt(dt, nvec) != 0;
}

bool hidden_lds_supported(int dt, int64_t cols) {
  if (cols % 4 != 0) return false;
  const int nvec = (int)(row_bytes(dt, cols) / 16);
  return (dt == 0 ? pick_nv_lds<0>(nvec) : dt == 1 ? pick_nv_lds<1>(nvec) : pick_nv_lds<2>(nvec)) != 0;
}

hipError_t launch_hidden_lds(const B1Gemv& g, hipStream_t s) {
  switch (g.dt) {
    case 0: return hidden_lds_dt<0>(g, s);
    case 1: return hidden_lds_dt<1>(g, s);
    default: return hidden_lds_dt<2>(g, s);
  }
}

hipError_t launch_fc1_b1(const B1Gemv& g, bool gated, hipStream_t s) {
  switch (g.dt) {
    case 0: return gated ? fc1_dt<0, true>(g, s) : fc1_dt<0, false>(g, s);
    case 1: return gated ? fc1_dt<1, true>(g, s) : fc1_dt<1, false>(g, s);
    default: return gated ? fc1_dt<2, true>(g, s) : fc1_dt<2, false>(g, s);
  }
}

bool pred_out_b1_supported(int pdt, int H, int N) {
  // buffer offsets into P2 are 32-bit
  return H >= 1 && H <= kMaxHiddenB1 && N >= 1 && (int64_t)H * row_bytes(pdt, N) < ((int64_t)1 << 31);
}

hipError_t launch_pred_out_b1(const PredFc1Args& a, hipStream_t s) {
  const bool b32 = a.c2 && a.c2_dt == PI_F32;
  switch (a.pdt) {
    case 0: return b32 ? pred_out_pdt<0, 0>(a, s) : pred_out_pdt<0, 1>(a, s);
    case 1: return b32 ? pred_out_pdt<1, 0>(a, s) : pred_out_pdt<1, 1>(a, s);
    default: return b32 ? pred_out_pdt<2, 0>(a, s) : pred_out_pdt<2, 1>(a, s);
  }
}

bool pred_fc1_supported(int pdt, int dt, int bdt, int c2dt, bool gated, int H, int N, int64_t d) {
  if (!pred_out_b1_supported(pdt, H, N)) return false;
  if (bdt != c2dt) return false;
  const int nvec = (int)(row_bytes(dt, d) / 16);
  const int nv = dt == 0 ? pick_nv_fused<0>(nvec) : dt == 1 ? pick_nv_fused<1>(nvec) : pick_nv_fused<2>(nvec);
  if (nv == 0) return false;
  if (pdt == 0 && dt == 0 && bdt == 0) return !gated;
  if (pdt == 1 && (dt == 1 || dt == 2) && bdt == 1) return true;
  if (pdt == 2 && dt == 1 && bdt == 1) return true;     // int4 predictor, fp16 FFN
  return false;
}

hipError_t launch_pred_fc1(const PredFc1Args& a, bool gated, hipStream_t s) {
  if (a.pdt == 0 && a.dt == 0) return pred_fc1_combo<0, 0, 0, false>(a, s);
  if (a.pdt == 1 && a.dt == 1) return gated ? pred_fc1_combo<1, 1, 1, true>(a, s) : pred_fc1_combo<1, 1, 1, false>(a, s);
  if (a.pdt == 1 && a.dt == 2) return gated ? pred_fc1_combo<1, 2, 1, true>(a, s) : pred_fc1_combo<1, 2, 1, false>(a, s);
  if (a.pdt == 2 && a.dt == 1) return gated ? pred_fc1_combo<2, 1, 1, true>(a, s) : pred_fc1_combo<2, 1, 1, false>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_fc2_seg(const Fc2SegArgs& a, hipStream_t s) {
  const int nbmax = (a.ngroups + kSegChunks - 1) / kSegChunks;
  const size_t shm = (size_t)nbmax * 64 * 4 * 2;
  const int tiles = seg_tiles(a.dt, a.d);
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

}  // namespace pi
