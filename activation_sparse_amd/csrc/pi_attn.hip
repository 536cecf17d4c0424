// pi_attn.hip - the self-attention block with head sparsity at decode (batch 1).
//
// A head predictor (the FFN predictor's two-layer MLP with one output per head)
// decides which heads run; every head's K and V entry for the new position goes
// to the fp16 cache (later tokens attend to it whatever this token's
// prediction), and only the predicted-active heads compute their query, attend
// over the cache and pass through the output projection.  Five launches, no
// workgroup waiting for another inside a launch:
//   k_attn_rows   : the predictor's hidden layer and the K and V projections, R
//                   rows per wave with x held in registers; K and V rounded to
//                   fp16 into the cache at position t
//   k_attn_q      : per workgroup of 8 waves (8 rows of one head), the head's
//                   logit (Pa2 row . g) and decision; the active heads' query
//                   rows, one per wave, x staged once in LDS
//   k_attn_part   : per (chunk of 64 cached positions, active head): scores,
//                   the chunk's max, exp2 weights, their sum and the weighted
//                   sum of the value rows
//   k_attn_out    : per (512-column tile, active head): the chunks combined in
//                   chunk order into o_h, then o_h times the head's rows of the
//                   transposed output projection over the tile
//   k_attn_reduce : y = bo + the active heads' tiles in head order; the
//                   ascending head list and its count
// Layouts: Wq, Wk, Wv [d x d], row r = output element r (head r / DH); WoT
// [d x d], row h*DH + i = the output-projection weights of head h's element i;
// Pa1 [Ha x d], Pa2 [n_heads x Ha]; caches [n_heads x L_max x DH] fp16, so a
// head's cached keys (values) are one contiguous run of 2*DH-byte rows.
#include "../../include/pi.h"
#include "pi_device.h"
#include "pi_attn.h"

namespace pi {
namespace {

constexpr int kAT = 256;                 // threads per workgroup
constexpr int kAW = kAT / kWave;         // waves per workgroup
constexpr int kRowsPerWave = 4;          // projection rows per wave (x loaded once)
constexpr int kChunk = 64;               // cached positions per attention workgroup
constexpr int kColTile = kWave * 8;      // output columns per k_attn_out workgroup (16-byte fp16 vectors)

__device__ __forceinline__ int wave_index() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave)); }

// x [d] into registers: lane's vectors v = u*64 + lane, 8 floats each (zeros past d).
template <int NV>
__device__ __forceinline__ void x_regs(const float* x, int nvec, int lane, float (&xr)[NV][8]) {
  const rsrc_t r = make_rsrc(uniform_ptr(x), (uint32_t)nvec * 32u);
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const uint32_t off = (uint32_t)(u * kWave + lane) * 32u;
    const uint4 a = bload16(r, off), b = bload16(r, off + 16u);
    xr[u][0] = __uint_as_float(a.x); xr[u][1] = __uint_as_float(a.y); xr[u][2] = __uint_as_float(a.z);
    xr[u][3] = __uint_as_float(a.w); xr[u][4] = __uint_as_float(b.x); xr[u][5] = __uint_as_float(b.y);
    xr[u][6] = __uint_as_float(b.z); xr[u][7] = __uint_as_float(b.w);
  }
}

// One fp16 row [d] dotted with the register x: all NV loads issued, then the fmas.
template <int NV>
__device__ __forceinline__ float row_dot(const void* row, int nvec, int lane, const float (&xr)[NV][8]) {
  const rsrc_t r = make_rsrc(uniform_ptr(row), row ? (uint32_t)nvec * 16u : 0u);
  uint4 w[NV];
#pragma unroll
  for (int u = 0; u < NV; ++u) w[u] = bload16(r, (uint32_t)(u * kWave + lane) * 16u);
  __builtin_amdgcn_sched_barrier(0);
  float acc = 0.f;
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    float wf[8];
    widen<1>(w[u], 1.f, wf);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf(wf[e], xr[u][e], acc);
  }
  return wave_sum(acc);
}

__device__ __forceinline__ uint16_t f2h_bits(float v) { return __builtin_bit_cast(uint16_t, (_Float16)v); }

// Rows [0, Ha): g = relu(Pa1 x + ca1); [Ha, Ha + d): K; [Ha + d, Ha + 2d): V.  Each wave takes
// kRowsPerWave consecutive rows of one kind (Ha and d are multiples of kRowsPerWave).
template <int NV>
__global__ __launch_bounds__(kAT) void k_attn_rows(AttnArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int r0 = (blockIdx.x * kAW + wave_index()) * kRowsPerWave;
  const int total = a.Ha + 2 * a.d;
  if (r0 >= total) return;
  const int nvec = a.d / 8;
  float xr[NV][8];
  x_regs<NV>(a.x, nvec, lane, xr);
  const Bias<1> ca1(a.ca1, (uint32_t)a.Ha), bk(a.bk, (uint32_t)a.d), bv(a.bv, (uint32_t)a.d);
#pragma unroll 1
  for (int k = 0; k < kRowsPerWave; ++k) {
    const int r = r0 + k;
    const char* row;
    float b;
    if (r < a.Ha) {
      row = static_cast<const char*>(a.Pa1) + (int64_t)r * a.d * 2;
      b = ca1(r);
    } else if (r < a.Ha + a.d) {
      row = static_cast<const char*>(a.Wk) + (int64_t)(r - a.Ha) * a.d * 2;
      b = bk(r - a.Ha);
    } else {
      row = static_cast<const char*>(a.Wv) + (int64_t)(r - a.Ha - a.d) * a.d * 2;
      b = bv(r - a.Ha - a.d);
    }
    const float z = row_dot<NV>(row, nvec, lane, xr) + b;
    if (lane == 0) {
      if (r < a.Ha) {
        a.g[r] = z > 0.f ? z : 0.f;
      } else {
        const int e = r < a.Ha + a.d ? r - a.Ha : r - a.Ha - a.d;
        const int h = e / a.dh, i = e % a.dh;
        uint16_t* c = r < a.Ha + a.d ? a.Kc : a.Vc;
        c[((int64_t)h * a.L_max + a.t) * a.dh + i] = f2h_bits(z);
      }
    }
  }
}

// Head h's logit from g: ca2[h] + Pa2[h] . g (Ha <= 1024: 16 per lane), the same bits in every wave.
__device__ __forceinline__ float head_logit(const AttnArgs& a, int h, int lane) {
  const rsrc_t rp = make_rsrc(uniform_ptr(static_cast<const char*>(a.Pa2) + (int64_t)h * a.Ha * 2), (uint32_t)a.Ha * 2u);
  const rsrc_t rg = make_rsrc(uniform_ptr(a.g), (uint32_t)a.Ha * 4u);
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int m = u * kWave + lane;
    const float w = h2f(bload2(rp, (uint32_t)m * 2u));
    const float gv = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rg, m * 4, 0, 0));
    s = fmaf(w, gv, s);
  }
  const Bias<1> ca2(a.ca2, (uint32_t)a.n_heads);
  return wave_sum(s) + ca2(h);
}

// Query rows: one row per wave, kQW waves per workgroup, all of one head.  Every wave computes its
// head's logit (the same bits) from the L2-resident Pa2 row and g while x streams in for LDS; an
// inactive head's workgroup leaves before any weight load, an active one issues its rows' loads,
// stores x to LDS, and the dots read x from there.  NV is the fewest 16-byte vectors per lane
// that cover a row, so no dead vector takes registers.  The head's first workgroup stores the
// logit and the decision.
constexpr int kQW = 8;
constexpr int kQRows = kQW;              // rows per workgroup
template <int NV>
__global__ __launch_bounds__(kQW * kWave) void k_attn_q(AttnArgs a) {
  extern __shared__ float4v xs[];
  const int lane = threadIdx.x & (kWave - 1), wave = wave_index();
  const int r = blockIdx.x * kQRows + wave;                   // d % kQRows == 0: every wave has a row
  const int h = (blockIdx.x * kQRows) / a.dh;                 // kQRows divides dh: one head per workgroup
  const int nvec = a.d / 8, nq = a.d / 4;
  float4v xv[4];
  {
    const rsrc_t rx = make_rsrc(uniform_ptr(a.x), (uint32_t)nq * 16u);
#pragma unroll
    for (int k = 0; k < 4; ++k) {                             // d <= 8192: at most 2048 float4, 4 per thread
      const uint4 t4 = bload16(rx, (uint32_t)(k * kQW * kWave + threadIdx.x) * 16u);
      xv[k] = float4v{__uint_as_float(t4.x), __uint_as_float(t4.y), __uint_as_float(t4.z), __uint_as_float(t4.w)};
    }
  }
  const float lg = head_logit(a, h, lane);
  const bool on = lg > a.tau;
  if ((blockIdx.x * kQRows) % a.dh == 0 && threadIdx.x == 0) {
    a.hlogit[h] = lg;
    a.flag[h] = on ? 1 : 0;
  }
  if (!on) return;                                            // the same decision in every wave
  const rsrc_t rw = make_rsrc(uniform_ptr(static_cast<const char*>(a.Wq) + (int64_t)r * a.d * 2), (uint32_t)nvec * 16u);
  uint4 w[NV];
#pragma unroll
  for (int u = 0; u < NV; ++u) w[u] = bload16(rw, (uint32_t)(u * kWave + lane) * 16u);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int q = k * kQW * kWave + threadIdx.x;
    if (q < nq) xs[q] = xv[k];
  }
  // zeros past the row's end, up to the NV * 64 vectors the dot reads (no index clamp, no select:
  // the weights there read zeros too)
  for (int q = nq + (int)threadIdx.x; q < 2 * NV * kWave; q += kQW * kWave) xs[q] = float4v{0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  // x is read from LDS one vector ahead of the dot (8 elements: float4 2v and 2v + 1), and each
  // vector's step closes with a scheduling barrier, so the reads are not all hoisted into registers
  float acc = 0.f;
  float4v xa0, xa1, xb0, xb1;
  auto xread = [&](int u, float4v& x0, float4v& x1) {
    const int v = u * kWave + lane;
    x0 = xs[2 * v];
    x1 = xs[2 * v + 1];
  };
  xread(0, xa0, xa1);
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    if (u + 1 < NV) xread(u + 1, xb0, xb1);
    float wf[8];
    widen<1>(w[u], 1.f, wf);
    acc = fmaf(wf[0], xa0.x, acc); acc = fmaf(wf[1], xa0.y, acc); acc = fmaf(wf[2], xa0.z, acc);
    acc = fmaf(wf[3], xa0.w, acc); acc = fmaf(wf[4], xa1.x, acc); acc = fmaf(wf[5], xa1.y, acc);
    acc = fmaf(wf[6], xa1.z, acc); acc = fmaf(wf[7], xa1.w, acc);
    __builtin_amdgcn_sched_barrier(0);
    xa0 = xb0; xa1 = xb1;
  }
  const Bias<1> bq(a.bq, (uint32_t)a.d);
  const float z = wave_sum(acc) + bq(r);
  if (lane == 0) a.q[r] = z;
}

// One chunk of kChunk cached positions of one active head.  LPP = DH/8 lanes per position (one
// 16-byte vector of 8 elements each), PPW = 64/LPP positions per wave-wide load, and each wave
// takes U = kChunk / (kAW * PPW) loads per lane.  Scores in the exp2 domain: e_j = q.K_j * log2(e) /
// sqrt(DH).  Writes m (the chunk's max score), l (sum of 2^(e_j - m)) and o (sum of 2^(e_j - m) V_j).
template <int DH>
__global__ __launch_bounds__(kAT) void k_attn_part(AttnArgs a) {
  constexpr int LPP = DH / 8, PPW = kWave / LPP, U = kChunk / (kAW * PPW);
  const int c = blockIdx.x, h = blockIdx.y;
  if (!a.flag[h]) return;
  __shared__ float s_max[kAW], s_sum[kAW];
  __shared__ float s_o[kAW][DH];
  const int lane = threadIdx.x & (kWave - 1), wave = wave_index();
  const int sub = lane % LPP, pg = lane / LPP;
  const int npos = a.t + 1;
  // the lane's 8 query elements
  float qv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) qv[e] = a.q[h * DH + sub * 8 + e];
  const uint32_t cbytes = (uint32_t)npos * DH * 2u;            // positions 0..t of this head
  const rsrc_t rk = make_rsrc(uniform_ptr(a.Kc + (int64_t)h * a.L_max * DH), cbytes);
  const rsrc_t rv = make_rsrc(uniform_ptr(a.Vc + (int64_t)h * a.L_max * DH), cbytes);
  uint4 kw[U], vw[U];
  int jpos[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    jpos[u] = c * kChunk + (u * kAW + wave) * PPW + pg;
    const uint32_t off = (uint32_t)jpos[u] * DH * 2u + (uint32_t)sub * 16u;   // past t: zeros, no request
    kw[u] = bload16(rk, off);
    vw[u] = bload16(rv, off);
  }
  __builtin_amdgcn_sched_barrier(0);
  const float sc = 1.4426950408889634f / sqrtf((float)DH);
  float ev[U];
  float mx = -INFINITY;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float kf[8];
    widen<1>(kw[u], 1.f, kf);
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s = fmaf(qv[e], kf[e], s);
#pragma unroll
    for (int off = LPP / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off, kWave);
    ev[u] = jpos[u] < npos ? s * sc : -INFINITY;
    mx = fmaxf(mx, ev[u]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, kWave));
  if (lane == 0) s_max[wave] = mx;
  __syncthreads();
  float m = s_max[0];
#pragma unroll
  for (int w = 1; w < kAW; ++w) m = fmaxf(m, s_max[w]);
  float l = 0.f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const float p = exp2f(ev[u] - m);                             // masked positions: 0
    float vf[8];
    widen<1>(vw[u], 1.f, vf);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = fmaf(p, vf[e], acc[e]);
    l += sub == 0 ? p : 0.f;                                      // one lane per position counts it
  }
  // over the position groups of the wave (lanes with the same sub), then over the waves
#pragma unroll
  for (int off = LPP; off < kWave; off <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], off, kWave);
  }
  l = wave_sum(l);
  if (pg == 0)
#pragma unroll
    for (int e = 0; e < 8; ++e) s_o[wave][sub * 8 + e] = acc[e];
  if (lane == 0) s_sum[wave] = l;
  __syncthreads();
  float* out = a.part + ((int64_t)h * a.n_chunks + c) * (DH + 2);
  if (threadIdx.x < DH) {
    float o = s_o[0][threadIdx.x];
#pragma unroll
    for (int w = 1; w < kAW; ++w) o += s_o[w][threadIdx.x];
    out[2 + threadIdx.x] = o;
  }
  if (threadIdx.x == 0) {
    float ls = s_sum[0];
#pragma unroll
    for (int w = 1; w < kAW; ++w) ls += s_sum[w];
    out[0] = m;
    out[1] = ls;
  }
}

// Head h's chunks combined in chunk order into o_h, then o_h times WoT rows h*DH .. h*DH + DH - 1
// over one tile of kColTile columns (the lane's 16-byte vector: 8 columns); the four waves take
// interleaved rows and are summed in wave order.
template <int DH>
__global__ __launch_bounds__(kAT) void k_attn_out(AttnArgs a) {
  constexpr int RW = DH / kAW;            // rows per wave
  const int tile = blockIdx.x, h = blockIdx.y;
  if (!a.flag[h]) return;
  __shared__ float s_o[DH];
  __shared__ float s_red[kAW][kColTile];
  const int lane = threadIdx.x & (kWave - 1), wave = wave_index();
  const float* ph = a.part + (int64_t)h * a.n_chunks * (DH + 2);
  const int nc = (a.t + 1 + kChunk - 1) / kChunk;
  // the combine's operands (from L2) are loaded before the weight rows (from HBM), so that the
  // in-order wait for them does not wait for the rows: up to kCombine chunks in registers
  constexpr int kCombine = 16;
  float cm[kCombine], cl[kCombine], co[kCombine];
  const int ti = threadIdx.x < DH ? threadIdx.x : 0;
#pragma unroll
  for (int c = 0; c < kCombine; ++c) {
    const bool in = c < nc;
    const int cc = in ? c : 0;                             // every address inside this head's chunks
    const float m = ph[cc * (DH + 2)], l = ph[cc * (DH + 2) + 1], o = ph[cc * (DH + 2) + 2 + ti];
    cm[c] = in ? m : -INFINITY;
    cl[c] = in ? l : 0.f;
    co[c] = in ? o : 0.f;
  }
  const int64_t col0 = (int64_t)tile * kColTile;
  const rsrc_t rw = make_rsrc(uniform_ptr(static_cast<const char*>(a.WoT) + ((int64_t)h * DH * a.d + col0) * 2),
                              (uint32_t)((int64_t)DH * a.d * 2 - col0 * 2));
  const bool vin = col0 + lane * 8 < a.d;
  uint4 w[RW];
#pragma unroll
  for (int k = 0; k < RW; ++k) {
    const int i = k * kAW + wave;
    w[k] = bload16(rw, vin ? (uint32_t)((int64_t)i * a.d * 2 + lane * 16) : 0xFFFFFFF0u);
  }
  __builtin_amdgcn_sched_barrier(0);
  if (threadIdx.x < DH) {
    float M = -INFINITY;
#pragma unroll
    for (int c = 0; c < kCombine; ++c) M = fmaxf(M, cm[c]);
    for (int c = kCombine; c < nc; ++c) M = fmaxf(M, ph[c * (DH + 2)]);
    float L = 0.f, o = 0.f;
#pragma unroll
    for (int c = 0; c < kCombine; ++c) {                  // chunk order; chunks past nc add 0
      const float f = c < nc ? exp2f(cm[c] - M) : 0.f;
      L = fmaf(cl[c], f, L);
      o = fmaf(co[c], f, o);
    }
    for (int c = kCombine; c < nc; ++c) {
      const float f = exp2f(ph[c * (DH + 2)] - M);
      L = fmaf(ph[c * (DH + 2) + 1], f, L);
      o = fmaf(ph[c * (DH + 2) + 2 + threadIdx.x], f, o);
    }
    s_o[threadIdx.x] = o / L;
  }
  __syncthreads();
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < RW; ++k) {
    const float ov = s_o[k * kAW + wave];
    float wf[8];
    widen<1>(w[k], 1.f, wf);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = fmaf(ov, wf[e], acc[e]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) s_red[wave][lane * 8 + e] = acc[e];
  __syncthreads();
  float* dst = a.ypart + (int64_t)h * a.d + col0;
  for (int cc = threadIdx.x; cc < kColTile; cc += kAT) {
    if (col0 + cc < a.d) {
      float s = s_red[0][cc];
#pragma unroll
      for (int ww = 1; ww < kAW; ++ww) s += s_red[ww][cc];
      dst[cc] = s;
    }
  }
}

// y = bo + the active heads' tiles in head order.  Each workgroup first lists the active heads in
// LDS (ascending, by ballots), then every thread issues its column's partials eight at a time;
// workgroup 0 also writes the list, its count and (optionally) the head logits.
__global__ __launch_bounds__(kAT) void k_attn_reduce(AttnArgs a) {
  __shared__ int s_list[kMaxAttnHeads];
  __shared__ int s_n;
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    int base = 0;
    for (int h0 = 0; h0 < a.n_heads; h0 += kWave) {
      const int h = h0 + lane;
      const bool on = h < a.n_heads && a.flag[h];
      const uint64_t bits = __ballot(on);
      const int pos = base + __popcll(bits & ((1ull << lane) - 1ull));
      if (on) {
        s_list[pos] = h;
        if (blockIdx.x == 0) a.heads[pos] = h;
      }
      if (blockIdx.x == 0 && a.logits_out && h < a.n_heads) a.logits_out[h] = a.hlogit[h];
      base += __popcll(bits);
    }
    if (lane == 0) {
      s_n = base;
      if (blockIdx.x == 0) *a.n_active = base;
    }
  }
  __syncthreads();
  const int64_t cidx = (int64_t)blockIdx.x * kAT + threadIdx.x;
  if (cidx >= a.d) return;
  const int n = s_n;
  float s = load_bias(a.bo, 1, cidx);
  for (int k0 = 0; k0 < n; k0 += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int hj = s_list[k0 + j < n ? k0 + j : n - 1];   // a listed head at every slot
      v[j] = a.ypart[(int64_t)hj * a.d + cidx];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (k0 + j < n) s += v[j];
  }
  a.y[cidx] = s;
}

int pick_nv_attn(int d) {
  const int nvec = d / 8;
  for (int nv : {1, 2, 4, 8, 16})
    if (nv * kWave >= nvec) return nv;
  return 0;
}

// The query kernel's 16-byte vectors per lane and row: the fewest that cover the row (two rows'
// loads are held at once, so no dead vector is carried).
int pick_nv_q(int d) {
  const int nvec = d / 8;
  for (int nv : {1, 2, 4, 6, 8, 10, 12, 14, 16})
    if (nv * kWave >= nvec) return nv;
  return 0;
}

template <int NV>
hipError_t launch_nv(const AttnArgs& a, hipStream_t s) {
  const int rows_blocks = (a.Ha + 2 * a.d + kAW * kRowsPerWave - 1) / (kAW * kRowsPerWave);
  hipLaunchKernelGGL(k_attn_rows<NV>, dim3((unsigned)rows_blocks), dim3(kAT), 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool attn_supported(int d, int n_heads, int dh, int Ha) {
  return (dh == 64 || dh == 128) && n_heads >= 1 && n_heads <= kMaxAttnHeads && d == n_heads * dh &&
         pick_nv_attn(d) != 0 && Ha >= kRowsPerWave && Ha <= 1024 && Ha % kRowsPerWave == 0;
}

int attn_chunks(int L_max) { return (L_max + kChunk - 1) / kChunk; }

hipError_t launch_attn(const AttnArgs& a, hipStream_t s) {
  hipError_t e;
  switch (pick_nv_attn(a.d)) {
    case 1: e = launch_nv<1>(a, s); break;
    case 2: e = launch_nv<2>(a, s); break;
    case 4: e = launch_nv<4>(a, s); break;
    case 8: e = launch_nv<8>(a, s); break;
    case 16: e = launch_nv<16>(a, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  {
    const dim3 gq((unsigned)(a.d / kQRows)), tq(kQW * kWave);
    const size_t shq = (size_t)pick_nv_q(a.d) * kWave * 32;   // x as 2 float4 per vector, NV * 64 vectors
    switch (pick_nv_q(a.d)) {
      case 1: hipLaunchKernelGGL(k_attn_q<1>, gq, tq, shq, s, a); break;
      case 2: hipLaunchKernelGGL(k_attn_q<2>, gq, tq, shq, s, a); break;
      case 4: hipLaunchKernelGGL(k_attn_q<4>, gq, tq, shq, s, a); break;
      case 6: hipLaunchKernelGGL(k_attn_q<6>, gq, tq, shq, s, a); break;
      case 8: hipLaunchKernelGGL(k_attn_q<8>, gq, tq, shq, s, a); break;
      case 10: hipLaunchKernelGGL(k_attn_q<10>, gq, tq, shq, s, a); break;
      case 12: hipLaunchKernelGGL(k_attn_q<12>, gq, tq, shq, s, a); break;
      case 14: hipLaunchKernelGGL(k_attn_q<14>, gq, tq, shq, s, a); break;
      default: hipLaunchKernelGGL(k_attn_q<16>, gq, tq, shq, s, a); break;
    }
  }
  const dim3 gp((unsigned)((a.t + 1 + kChunk - 1) / kChunk), (unsigned)a.n_heads);
  const dim3 go((unsigned)((a.d + kColTile - 1) / kColTile), (unsigned)a.n_heads);
  if (a.dh == 128) {
    hipLaunchKernelGGL(k_attn_part<128>, gp, dim3(kAT), 0, s, a);
    hipLaunchKernelGGL(k_attn_out<128>, go, dim3(kAT), 0, s, a);
  } else {
    hipLaunchKernelGGL(k_attn_part<64>, gp, dim3(kAT), 0, s, a);
    hipLaunchKernelGGL(k_attn_out<64>, go, dim3(kAT), 0, s, a);
  }
  hipLaunchKernelGGL(k_attn_reduce, dim3((unsigned)((a.d + kAT - 1) / kAT)), dim3(kAT), 0, s, a);
  return hipGetLastError();
}

}  // namespace pi
