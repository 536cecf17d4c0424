// pi_generic.hip - libpi kernels for any batch size and row length (gfx950, wave64).
//
//  k_rowdot  : row-dot GEMV over dense rows (predictor layers) or over the
//              rows listed in the active list (FC1), fused bias + ReLU (and
//              the gate * up product of a gated FFN).  One wave per row, 16-B
//              loads along the row, fp32 accumulate, x staged in LDS.
//  k_compact : threshold + union over the batch + wave ballot + block prefix
//              sum -> ascending slot list and its count (stays on device).
//  k_merge   : y += y_c (+ b2), skipped on the device when no cold neuron is
//              active.
//  k_layer_norm : chained layers; one layer's output row normalised (mean 0,
//              unit variance) into the next layer's input.  One workgroup per
//              row, 16-byte loads, the row held in registers up to 16 Ki
//              elements.
#include "pi_device.h"
#include "pi_internal.h"
#include "pi_list.h"

namespace pi {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;
constexpr int kXsMaxBytes = 64 * 1024;

template <int DT, int NB, bool GATED>
__global__ __launch_bounds__(kThreads) void k_rowdot(RowdotArgs a, int64_t n_rows, int stage_x,
                                                      uint32_t* zero_ptr, int zero_n) {
  constexpr int E = Fmt<DT>::E;
  extern __shared__ float xs[];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  if (zero_ptr && blockIdx.x == 0)
    for (int t = tid; t < zero_n; t += kThreads) zero_ptr[t] = 0u;
  const int64_t cols = a.cols;
  const int B = a.B;
  const float* xp = a.x;
  if (stage_x) {
    const int64_t n4 = (int64_t)B * cols / 4;
    const float4v* src = reinterpret_cast<const float4v*>(a.x);
    float4v* dst = reinterpret_cast<float4v*>(xs);
    for (int64_t t = tid; t < n4; t += kThreads) dst[t] = src[t];
    __syncthreads();
    xp = xs;
  }
  int64_t count = a.count_max;
  if (a.list) {
    int64_t kd = *a.count_dev;
    count = kd < 0 ? 0 : (kd < a.count_max ? kd : a.count_max);
  }
  const int64_t rb = row_bytes(DT, cols);
  const int nvec = (int)(rb / 16);
  const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + wave;
  const int64_t nw = (int64_t)gridDim.x * kWavesPerBlock;
  const int64_t groups = cols / 128;
  for (int64_t j = gw; j < count; j += nw) {
    const int64_t row = a.list ? (int64_t)a.list[j] : j;
    float acc[NB], acc2[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) { acc[b] = 0.f; acc2[b] = 0.f; }
    const bool row_ok = row >= 0 && row < n_rows;
    if (row_ok) {
      const char* rp = reinterpret_cast<const char*>(a.W) + row * rb;
      const char* up = GATED ? reinterpret_cast<const char*>(a.Wup) + row * rb : nullptr;
#pragma unroll 4
      for (int v = lane; v < nvec; v += kWave) {
        float wf[E], uf[E];
        float sc = 1.f, scu = 1.f;
        if constexpr (DT == 2) {
          sc = h2f(a.Ws[row * groups + v / 4]);
          if constexpr (GATED) scu = h2f(a.Wups[row * groups + v / 4]);
        }
        widen<DT>(ld16(rp + (int64_t)v * 16), sc, wf);
        if constexpr (GATED) widen<DT>(ld16(up + (int64_t)v * 16), scu, uf);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          if (b < B) {
            const float* xb = xp + (int64_t)b * cols + (int64_t)v * E;
#pragma unroll
            for (int e = 0; e < E; ++e) {
              acc[b] = fmaf(wf[e], xb[e], acc[b]);
              if constexpr (GATED) acc2[b] = fmaf(uf[e], xb[e], acc2[b]);
            }
          }
        }
      }
    }
    const float bias = row_ok ? load_bias(a.bias, a.bias_dt, row) : 0.f;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b < B) {
        float z = wave_sum(acc[b]) + bias;
        if (a.relu) z = z > 0.f ? z : 0.f;
        if constexpr (GATED) z *= wave_sum(acc2[b]);
        if (!row_ok) z = 0.f;
        if (lane == 0) a.out[(int64_t)b * a.out_stride + j] = z;
      }
    }
  }
}

constexpr int kCompactThreads = 1024;
constexpr int kCompactWaves = kCompactThreads / kWave;   // 16
constexpr int kCompactLogits = 32;                       // logit loads in flight per lane: 32768 ids per round
constexpr int kCompactBelow = 16;                        // table loads in flight per lane for the count below c0
constexpr int kCompactOwn = 2;                           // own slots per lane (chunk <= 2 * kCompactThreads)

// Standalone compaction over any table order, in blocks that wait for no other
// and keep their global loads in flight together (the stage sits between two
// dependent launches, so its latency is what counts): block (c, t) owns slots
// [c0, c1) of table t (0: GPU, 1: CPU).  It issues the table loads of its own
// slots and of the first slots below c0, rebuilds every activation word in LDS
// from the logits (union over the batch, one wave ballot per 64 ids), counts
// the table's active slots below c0, and writes its own active slots in
// ascending order at that offset (wave ballot + block prefix sum per pass of
// kCompactThreads slots).  The block owning the last slot writes the count.
__global__ __launch_bounds__(kCompactThreads) void k_compact(int B, int N, const float* __restrict__ logits,
                                                             float tau, const int32_t* T_g, int n_g,
                                                             int32_t* A_g, int32_t* K_g, const int32_t* T_c,
                                                             int n_c, int32_t* A_c, int32_t* K_c, int chunk) {
  const int32_t* T = blockIdx.y == 0 ? T_g : T_c;
  const int n = blockIdx.y == 0 ? n_g : n_c;
  int32_t* A = blockIdx.y == 0 ? A_g : A_c;
  int32_t* Kout = blockIdx.y == 0 ? K_g : K_c;
  const int c0 = (int)blockIdx.x * chunk;
  if (c0 >= n && !(c0 == 0 && n == 0)) return;            // past the table (block-uniform)
  const int c1 = c0 + chunk < n ? c0 + chunk : n;
  extern __shared__ uint64_t words[];                      // ceil(N / 64)
  __shared__ int wtot[kCompactWaves];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  const int nw = (N + 63) / 64;
  // table ids: own slots (at most kCompactOwn passes) and the first round below c0
  int own[kCompactOwn], low[kCompactBelow];
#pragma unroll
  for (int q = 0; q < kCompactOwn; ++q) {
    const int s = c0 + q * kCompactThreads + tid;
    own[q] = s < c1 ? T[s] : -1;
  }
#pragma unroll
  for (int q = 0; q < kCompactBelow; ++q) {
    const int s = q * kCompactThreads + tid;
    low[q] = s < c0 ? T[s] : -1;
  }
  // 1. the activation words: group g of 64 ids is wave (g / kCompactLogits) % kCompactWaves's
  for (int g0 = wv * kCompactLogits; g0 < nw; g0 += kCompactWaves * kCompactLogits) {
    uint32_t f = 0;                                        // bit q: group g0 + q active at this lane
    for (int b = 0; b < B; ++b) {
      const float* row = logits + (int64_t)b * N;
      float z[kCompactLogits];
#pragma unroll
      for (int q = 0; q < kCompactLogits; ++q) {
        const int id = (g0 + q) * 64 + lane;
        z[q] = id < N ? row[id] : tau;
      }
#pragma unroll
      for (int q = 0; q < kCompactLogits; ++q) f |= (z[q] > tau ? 1u : 0u) << q;
    }
#pragma unroll
    for (int q = 0; q < kCompactLogits; ++q) {
      const uint64_t w = __ballot((f >> q) & 1u);
      if (lane == 0 && g0 + q < nw) words[g0 + q] = w;
    }
  }
  __syncthreads();
  auto bit = [&](int id) { return id >= 0 && id < N && ((words[id >> 6] >> (id & 63)) & 1ull); };
  // 2. active slots below c0
  int below = 0;
#pragma unroll
  for (int q = 0; q < kCompactBelow; ++q) below += bit(low[q]) ? 1 : 0;
  for (int s0 = kCompactBelow * kCompactThreads + tid; s0 < c0; s0 += kCompactThreads * kCompactBelow) {
#pragma unroll
    for (int q = 0; q < kCompactBelow; ++q) {
      const int s = s0 + q * kCompactThreads;
      low[q] = s < c0 ? T[s] : -1;
    }
#pragma unroll
    for (int q = 0; q < kCompactBelow; ++q) below += bit(low[q]) ? 1 : 0;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) below += __shfl_xor(below, off, kWave);
  if (lane == 0) wtot[wv] = below;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < kCompactWaves; ++w) base += wtot[w];
  __syncthreads();
  // 3. this block's slots, ascending
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int q = 0; q < kCompactOwn; ++q) {
    if (c0 + q * kCompactThreads >= c1) break;              // block-uniform
    const bool f = bit(own[q]);
    const uint64_t bal = __ballot(f);
    if (lane == 0) wtot[wv] = __popcll(bal);
    __syncthreads();
    int pre = 0, tot = 0;
    for (int w = 0; w < kCompactWaves; ++w) {
      if (w < wv) pre += wtot[w];
      tot += wtot[w];
    }
    if (f) A[base + pre + __popcll(bal & lt_mask)] = c0 + q * kCompactThreads + tid;
    base += tot;
    __syncthreads();
  }
  if (c1 == n && tid == 0) *Kout = base;
}

// Streaming read: 256 threads per block, grid-stride over 16-byte vectors,
// D loads per lane in flight; each wave's XOR of what it read is stored.
template <int D>
__global__ __launch_bounds__(256) void k_read_probe(const uint4* __restrict__ p, int64_t n16, uint32_t* out) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (D - 1) * stride < n16; i += D * stride) {
    uint4 v[D];
#pragma unroll
    for (int q = 0; q < D; ++q) v[q] = p[i + q * stride];
#pragma unroll
    for (int q = 0; q < D; ++q) acc ^= v[q].x ^ v[q].y ^ v[q].z ^ v[q].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off, kWave);
  if ((threadIdx.x & (kWave - 1)) == 0) out[blockIdx.x * 4 + threadIdx.x / kWave] = acc;
}

constexpr int kLnThreads = 1024;
constexpr int kLnReg = 16;   // elements per thread held in registers: rows up to 16 Ki

// Sum over the workgroup in a fixed order: butterfly within each wave, then the
// waves' sums in wave order.  Every thread returns the same value.
__device__ __forceinline__ float ln_block_sum(float v, float* red) {
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kLnThreads / kWave; ++i) s += red[i];
  __syncthreads();          // red is reused by the next sum
  return s;
}

template <int V>
__device__ __forceinline__ void ln_load(const float* p, float* e) {
  if constexpr (V == 4) {
    const float4 q = *reinterpret_cast<const float4*>(p);
    e[0] = q.x; e[1] = q.y; e[2] = q.z; e[3] = q.w;
  } else {
    e[0] = *p;
  }
}

template <int V>
__device__ __forceinline__ void ln_store(float* p, const float* e) {
  if constexpr (V == 4) *reinterpret_cast<float4*>(p) = make_float4(e[0], e[1], e[2], e[3]);
  else *p = e[0];
}

// x[b,:] = (y[b,:] - mean) / sqrt(var + eps), population variance.  V = 4:
// 16-byte loads and stores (d % 4 == 0, aligned rows), else single floats.
// Rows past what the registers hold are read again from memory in each pass.
// Each element is read and written by one thread, after both sums: x may be y.
template <int V>
__global__ __launch_bounds__(kLnThreads) void k_layer_norm(int d, const float* y, float eps, float* x) {
  constexpr int G = kLnReg / V;             // loads per thread held in registers
  __shared__ float red[kLnThreads / kWave];
  const float* r = y + (int64_t)blockIdx.x * d;
  float* o = x + (int64_t)blockIdx.x * d;
  const int t = threadIdx.x, ng = d / V;
  const bool held = ng <= G * kLnThreads;
  float v[G][V];
  float s = 0.f;
  if (held) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int q = t + j * kLnThreads;
      if (q < ng) {
        ln_load<V>(r + (int64_t)q * V, v[j]);
      } else {
#pragma unroll
        for (int e = 0; e < V; ++e) v[j][e] = 0.f;
      }
    }
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int e = 0; e < V; ++e) s += v[j][e];
  } else {
    for (int q = t; q < ng; q += kLnThreads) {
      float e4[V];
      ln_load<V>(r + (int64_t)q * V, e4);
#pragma unroll
      for (int e = 0; e < V; ++e) s += e4[e];
    }
  }
  const float mu = ln_block_sum(s, red) / (float)d;
  float sq = 0.f;
  if (held) {
#pragma unroll
    for (int j = 0; j < G; ++j)
      if (t + j * kLnThreads < ng) {
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const float dv = v[j][e] - mu;
          sq += dv * dv;
        }
      }
  } else {
    for (int q = t; q < ng; q += kLnThreads) {
      float e4[V];
      ln_load<V>(r + (int64_t)q * V, e4);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float dv = e4[e] - mu;
        sq += dv * dv;
      }
    }
  }
  const float var = ln_block_sum(sq, red) / (float)d;
  const float inv = 1.0f / sqrtf(var + eps);
  if (held) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int q = t + j * kLnThreads;
      if (q < ng) {
        float e4[V];
#pragma unroll
        for (int e = 0; e < V; ++e) e4[e] = (v[j][e] - mu) * inv;
        ln_store<V>(o + (int64_t)q * V, e4);
      }
    }
  } else {
    for (int q = t; q < ng; q += kLnThreads) {
      float e4[V];
      ln_load<V>(r + (int64_t)q * V, e4);
#pragma unroll
      for (int e = 0; e < V; ++e) e4[e] = (e4[e] - mu) * inv;
      ln_store<V>(o + (int64_t)q * V, e4);
    }
  }
}

__global__ __launch_bounds__(kThreads) void k_merge(int64_t n, int d, float* y, const float* y_c,
                                                    const int32_t* K_c, const void* b2, int b2_dt) {
  const bool add_c = y_c && (!K_c || *K_c != 0);
  if (!add_c && !b2) return;
  for (int64_t t = blockIdx.x * (int64_t)kThreads + threadIdx.x; t < n; t += (int64_t)gridDim.x * kThreads) {
    float v = y[t];
    if (add_c) v += y_c[t];
    if (b2) v += load_bias(b2, b2_dt, t % d);
    y[t] = v;
  }
}

// Union activation words from stored logits [B x N]: one wave per 64 ids.
// Lists from activation words + prepared table; each block writes a strided
// share of A_g and A_c, block 0 the counts.
__global__ __launch_bounds__(kThreads) void k_list(ListCtx c) {
  extern __shared__ uint32_t lsm[];
  const ListView v = list_build<kThreads>(c, lsm);
  for (int j = blockIdx.x * kThreads + threadIdx.x; j < v.K; j += gridDim.x * kThreads) c.A_g[j] = list_slot(v, j);
  list_write_cold_and_counts<kThreads>(c, v);
}

__global__ void k_zero_u32(uint32_t* p, int64_t n) {
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < n; t += (int64_t)gridDim.x * blockDim.x) p[t] = 0u;
}

template <int DT, bool GATED>
hipError_t rowdot_dt(const RowdotArgs& a, int64_t n_rows, uint32_t* zero_ptr, int zero_n, hipStream_t s) {
  const int64_t xbytes = (int64_t)a.B * a.cols * 4;
  const int stage = xbytes <= kXsMaxBytes;
  const size_t shm = stage ? (size_t)xbytes : 0;
  int64_t blocks = (a.count_max + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks > 2048) blocks = 2048;
  if (blocks < 1) blocks = 1;
  dim3 g((unsigned)blocks), t(kThreads);
  if (a.B <= 1) hipLaunchKernelGGL((k_rowdot<DT, 1, GATED>), g, t, shm, s, a, n_rows, stage, zero_ptr, zero_n);
  else if (a.B <= 2) hipLaunchKernelGGL((k_rowdot<DT, 2, GATED>), g, t, shm, s, a, n_rows, stage, zero_ptr, zero_n);
  else if (a.B <= 4) hipLaunchKernelGGL((k_rowdot<DT, 4, GATED>), g, t, shm, s, a, n_rows, stage, zero_ptr, zero_n);
  else if (a.B <= 8) hipLaunchKernelGGL((k_rowdot<DT, 8, GATED>), g, t, shm, s, a, n_rows, stage, zero_ptr, zero_n);
  else if (a.B <= 16) hipLaunchKernelGGL((k_rowdot<DT, 16, GATED>), g, t, shm, s, a, n_rows, stage, zero_ptr, zero_n);
  else hipLaunchKernelGGL((k_rowdot<DT, 32, GATED>), g, t, shm, s, a, n_rows, stage, zero_ptr, zero_n);
  return hipGetLastError();
}

}  // namespace

// n_rows: rows in the matrix (bound for listed row ids).  For dense mode it
// equals count_max.  zero_ptr/zero_n: u32 words block 0 clears first (the FC2
// tile counters), or NULL.
hipError_t launch_rowdot_ex(const RowdotArgs& a, int64_t n_rows, uint32_t* zero_ptr, int zero_n, hipStream_t s) {
  if (a.gated) {
    switch (a.dt) {
      case PI_F32: return rowdot_dt<0, true>(a, n_rows, zero_ptr, zero_n, s);
      case PI_F16: return rowdot_dt<1, true>(a, n_rows, zero_ptr, zero_n, s);
      default: return rowdot_dt<2, true>(a, n_rows, zero_ptr, zero_n, s);
    }
  }
  switch (a.dt) {
    case PI_F32: return rowdot_dt<0, false>(a, n_rows, zero_ptr, zero_n, s);
    case PI_F16: return rowdot_dt<1, false>(a, n_rows, zero_ptr, zero_n, s);
    default: return rowdot_dt<2, false>(a, n_rows, zero_ptr, zero_n, s);
  }
}

hipError_t launch_rowdot(const RowdotArgs& a, hipStream_t s) { return launch_rowdot_ex(a, a.count_max, nullptr, 0, s); }

hipError_t launch_compact(int B, int N, const float* logits, float tau, const int32_t* T_g, int n_g,
                          int32_t* A_g, int32_t* K, const int32_t* T_c, int n_c, int32_t* A_c,
                          int32_t* K_c, hipStream_t s) {
  // whole passes of slots per block, at most kCompactOwn of them (up to 32 blocks per table at
  // PI_MAX_NEURONS)
  const int nmax = n_g > n_c ? n_g : n_c;
  const int chunk = nmax > 32 * kCompactThreads ? kCompactOwn * kCompactThreads : kCompactThreads;
  const int blocks = (nmax + chunk - 1) / chunk > 0 ? (nmax + chunk - 1) / chunk : 1;
  const size_t shm = (size_t)((N + 63) / 64) * 8;
  hipLaunchKernelGGL(k_compact, dim3((unsigned)blocks, T_c ? 2u : 1u), dim3(kCompactThreads), shm, s, B, N, logits,
                     tau, T_g, n_g, A_g, K, T_c, n_c, A_c, K_c, chunk);
  return hipGetLastError();
}

hipError_t launch_read_probe(const void* buf, int64_t bytes, int blocks, int depth, uint32_t* out, hipStream_t s) {
  const uint4* p = static_cast<const uint4*>(buf);
  const dim3 g((unsigned)blocks), t(256);
  switch (depth) {
    case 4: hipLaunchKernelGGL(k_read_probe<4>, g, t, 0, s, p, bytes / 16, out); break;
    case 8: hipLaunchKernelGGL(k_read_probe<8>, g, t, 0, s, p, bytes / 16, out); break;
    case 16: hipLaunchKernelGGL(k_read_probe<16>, g, t, 0, s, p, bytes / 16, out); break;
    case 32: hipLaunchKernelGGL(k_read_probe<32>, g, t, 0, s, p, bytes / 16, out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_list(const ListCtx& c, int n_g, hipStream_t s) {
  int blocks = (n_g + kThreads - 1) / kThreads;
  blocks = blocks < 1 ? 1 : (blocks > 64 ? 64 : blocks);
  hipLaunchKernelGGL(k_list, dim3((unsigned)blocks), dim3(kThreads), (size_t)list_smem_words(c.W) * 4, s, c);
  return hipGetLastError();
}

hipError_t launch_zero_u32(uint32_t* p, int64_t n, hipStream_t s) {
  hipLaunchKernelGGL(k_zero_u32, dim3(1), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_layer_norm(int B, int d, const float* y, float eps, float* x, hipStream_t s) {
  const bool vec = d % 4 == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0;
  if (vec) hipLaunchKernelGGL(k_layer_norm<4>, dim3((unsigned)B), dim3(kLnThreads), 0, s, d, y, eps, x);
  else hipLaunchKernelGGL(k_layer_norm<1>, dim3((unsigned)B), dim3(kLnThreads), 0, s, d, y, eps, x);
  return hipGetLastError();
}

hipError_t launch_merge(int B, int d, float* y, const float* y_c, const int32_t* K_c, const void* b2, int b2_dt,
                        hipStream_t s) {
  const int64_t n = (int64_t)B * d;
  int64_t blocks = (n + kThreads - 1) / kThreads;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(k_merge, dim3((unsigned)blocks), dim3(kThreads), 0, s, n, d, y, y_c, K_c, b2, b2_dt);
  return hipGetLastError();
}

}  // namespace pi
