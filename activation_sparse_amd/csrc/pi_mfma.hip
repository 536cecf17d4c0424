// pi_mfma.hip - the batched GEMMs on the matrix cores.
//
// fp16 weights (every layer of the fp16 configurations) run on the fp16
// instruction v_mfma_f32_16x16x32_f16, whose products of two fp16 values are
// exact and accumulate in fp32:
//  * FC1: x is rounded to fp16 (k_mm_rowdot16);
//  * FC2: the activations a are fp16, written so by the FC1 finish;
//  * the predictor's two layers keep near-fp32 operands as two fp16 parts,
//    hi + lo (about 22 bits), with two exact products per weight: x for the
//    hidden layer (k_mm_rowdot16 with HILO), h for the output layer
//    (k_mm_axpy16 with LO), so the logits stay inside the activation
//    decision's parity band.
// Other weight types (fp32, int4 groups) keep the fp32-input instruction
// v_mfma_f32_16x16x4_f32: the weights are widened to fp32 in registers, x, h
// and a stay fp32, and the arithmetic is the VALU path's with the operand
// reuse of a matrix tile (k_mm_rowdot, k_mm_axpy).
//
// One 16x16x4 instruction sums over k = 4 lane groups g = lane / 16.  Each lane
// loads one 16-byte weight vector (E consecutive elements along k) and feeds
// them to E consecutive instructions: at step s the lane group g supplies
// k = kb + E*g + s, so E instructions cover the kb .. kb + 4E block once.
//
//  k_mm_rowdot : out[pos, b] = sum_k W[row(pos), k] * x[b, k] over a k-chunk
//                (predictor hidden layer: dense rows; FC1: the listed rows).
//                Tile 16 rows x 16*NBT batch rows per wave, split-K partials.
//  k_mm_finish : sums the split-K partials in chunk order, + bias, ReLU
//                (x the up product for a gated FFN) -> [B x stride].
//  k_mm_axpy   : out[b, c] = sum_j a[b, j] * W[row(j), c] over a row chunk
//                (predictor output layer over hidden-major P2: dense rows;
//                FC2: the listed rows).  A lane's 16-byte row vector holds
//                columns c0 + E*n + e (n = lane % 16): column tile e of the
//                wave's 16E columns, so one load feeds E instructions.  The
//                block's four waves take interleaved row steps and are summed
//                in LDS in wave order; one partial per (row chunk, b, c).
#include "pi_device.h"
#include "pi_internal.h"

namespace pi {
namespace {

typedef float float4v_t __attribute__((ext_vector_type(4)));

constexpr int kMmWaves = 4;
constexpr int kMmThreads = kMmWaves * kWave;
constexpr int kOutWaves = 8;   // the predictor output layer's one-row-chunk axpy (k_mm_axpy16)
// its row ids take 4 bytes each of dynamic LDS beside the waves' sums; it is measured up to this
// many hidden units (more than any predictor here), and past them the four-wave block takes the layer
constexpr int64_t kOutWavesMaxRows = 16384;

__device__ __forceinline__ float4v_t mfma4(float a, float b, float4v_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// E weights of one 16-byte vector, widened (int4: times its group scale).
template <int DT>
__device__ __forceinline__ void widen_vec(uint4 v, float scale, float* out) {
  widen<DT>(v, scale, out);
}

template <int DT, int NBT, bool GATED>
__global__ __launch_bounds__(kMmThreads) void k_mm_rowdot(MmRowArgs a) {
  constexpr int E = Fmt<DT>::E;
  constexpr int KB = 4 * E;                 // k per block of E instructions
  constexpr int D = DT == 2 ? 1 : 4;        // k blocks in flight
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int tile = blockIdx.x * kMmWaves + wave;
  const int ks = blockIdx.y;
  int64_t count = a.count_max;
  if (a.list) {
    const int64_t kd = *a.count_dev;
    count = kd < 0 ? 0 : (kd < a.count_max ? kd : a.count_max);
  }
  if ((int64_t)tile * 16 >= count) return;
  const int g = lane / 16, ml = lane % 16;
  // A operand row of this lane
  const int64_t pos = (int64_t)tile * 16 + ml;
  const bool pin = pos < count;
  int64_t row = pin ? (a.list ? (int64_t)a.list[pos] : pos) : -1;
  if (row >= a.n_rows) row = -1;
  const int64_t rb = row_bytes(DT, a.cols);
  const int64_t groups = a.cols / 128;
  const char* W = reinterpret_cast<const char*>(a.W);
  const char* Wu = reinterpret_cast<const char*>(a.Wup);
  // one buffer over the whole matrix (the host keeps it below 2^31 bytes);
  // an absent row reads zeros
  const uint32_t wbytes = (uint32_t)(a.n_rows * rb);
  const rsrc_t rW = make_rsrc(W, wbytes);
  const rsrc_t rU = make_rsrc(GATED ? Wu : W, GATED ? wbytes : 0u);
  const rsrc_t rS = make_rsrc(DT == 2 ? (const void*)a.Ws : W, DT == 2 ? (uint32_t)(a.n_rows * groups * 2) : 0u);
  const rsrc_t rSu = make_rsrc(DT == 2 && GATED ? (const void*)a.Wups : W, DT == 2 && GATED ? (uint32_t)(a.n_rows * groups * 2) : 0u);
  const uint32_t roff = row >= 0 ? (uint32_t)(row * rb) : 0u;
  const uint32_t soff = row >= 0 ? (uint32_t)(row * groups * 2) : 0u;
  // B operand: x rows b = 16 t + lane % 16 (zeros past B)
  const rsrc_t rX = make_rsrc(a.x, (uint32_t)(a.B * a.cols * 4));
  uint32_t xoff[NBT];
  bool xok[NBT];
#pragma unroll
  for (int t = 0; t < NBT; ++t) {
    const int b = 16 * t + ml;
    xok[t] = b < a.B;
    xoff[t] = xok[t] ? (uint32_t)(b * a.cols * 4) : 0u;
  }
  // every load whose predicate fails takes this offset, past every range
  constexpr uint32_t kOut = 0xFFFFFFF0u;
  const int64_t k0 = (int64_t)ks * a.kc, k1 = k0 + a.kc < a.cols ? k0 + a.kc : a.cols;
  float4v_t acc[NBT], accu[NBT];
#pragma unroll
  for (int t = 0; t < NBT; ++t) {
    acc[t] = float4v_t{0.f, 0.f, 0.f, 0.f};
    accu[t] = float4v_t{0.f, 0.f, 0.f, 0.f};
  }
  for (int64_t kb = k0; kb < k1; kb += (int64_t)D * KB) {
    uint4 wv[D], uv[D];
    float sc[D], scu[D];
    float4v xv[D][NBT][E / 4];
#pragma unroll
    for (int i = 0; i < D; ++i) {
      const int64_t kk = kb + (int64_t)i * KB + (int64_t)E * g;   // this lane's first k
      const bool kin = kb + (int64_t)i * KB < k1;                  // whole blocks: cols % KB == 0
      const bool wok = kin && row >= 0;
      const uint32_t eoff = (uint32_t)(row_bytes(DT, kk));
      wv[i] = bload16(rW, wok ? roff + eoff : kOut);
      if constexpr (GATED) uv[i] = bload16(rU, wok ? roff + eoff : kOut);
      if constexpr (DT == 2) {
        sc[i] = h2f(bload2(rS, wok ? soff + (uint32_t)(kk / 128) * 2u : kOut));
        if constexpr (GATED) scu[i] = h2f(bload2(rSu, wok ? soff + (uint32_t)(kk / 128) * 2u : kOut));
      }
#pragma unroll
      for (int t = 0; t < NBT; ++t)
#pragma unroll
        for (int q = 0; q < E / 4; ++q) {
          const uint4 v = bload16(rX, kin && xok[t] ? xoff[t] + (uint32_t)(kk * 4 + 16 * q) : kOut);
          xv[i][t][q] = float4v{__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w)};
        }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < D; ++i) {
      float wf[E], uf[E];
      widen_vec<DT>(wv[i], DT == 2 ? sc[i] : 1.f, wf);
      if constexpr (GATED) widen_vec<DT>(uv[i], DT == 2 ? scu[i] : 1.f, uf);
#pragma unroll
      for (int s = 0; s < E; ++s) {
#pragma unroll
        for (int t = 0; t < NBT; ++t) {
          const float xs = xv[i][t][s / 4][s % 4];
          acc[t] = mfma4(wf[s], xs, acc[t]);
          if constexpr (GATED) accu[t] = mfma4(uf[s], xs, accu[t]);
        }
      }
    }
  }
  // D[m = 4g + r][n = lane % 16]: row position tile*16 + 4g + r, batch 16t + lane % 16
  const int NBP = 16 * NBT;
#pragma unroll
  for (int t = 0; t < NBT; ++t) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t p = (int64_t)tile * 16 + 4 * g + r;
      if (p < count) {
        const int64_t o = ((int64_t)ks * a.count_max + p) * NBP + 16 * t + ml;
        a.partials[o] = acc[t][r];
        if constexpr (GATED) a.partials[(int64_t)a.ks * a.count_max * NBP + o] = accu[t][r];
      }
    }
  }
}

// fp16 weights with x rounded to fp16 (FC1 of the batched path): one
// v_mfma_f32_16x16x32_f16 per 32 k takes the lane's 16-byte weight vector as
// it is (row m = lane % 16, k = 8 g .. 8 g + 7, g = lane / 16) and 8 fp16 x of
// batch row lane % 16 at the same k, accumulating in fp32.  The block's four
// waves share one k chunk: x[16 nbt][chunk] is rounded to fp16 once, into LDS
// (rows padded by 16 bytes, so the 16 lanes of a lane group hit distinct banks).
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
// waves per block, sharing the block's x chunk (more for 32 batch rows, whose chunk is twice the size)
constexpr int r16_waves(int nbt) { return nbt == 1 ? 4 : 16; }
// largest k chunk: x[16 nbt][chunk] in fp16 within 64 KB of LDS (two such planes with hi / lo x)
constexpr int row16_kcmax(int nbt, bool hilo = false) { return hilo ? (nbt == 1 ? 992 : 480) : (nbt == 1 ? 1024 : 960); }

__device__ __forceinline__ float4v_t mfma16(half8_t a, half8_t b, float4v_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

template <int NBT, bool GATED, bool HILO>
__global__ __launch_bounds__(r16_waves(NBT) * kWave) void k_mm_rowdot16(MmRowArgs a) {
  constexpr int WPB = r16_waves(NBT), NT = WPB * kWave;
  constexpr int D = 8;                      // k blocks of 32 in flight
  extern __shared__ __attribute__((aligned(16))) _Float16 xh[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  int64_t count = a.count_max;
  if (a.list) {
    const int64_t kd = *a.count_dev;
    count = kd < 0 ? 0 : (kd < a.count_max ? kd : a.count_max);
  }
  if ((int64_t)blockIdx.x * WPB * 16 >= count) return;   // the whole block: before the barrier
  const int NBP = 16 * NBT;
  const int64_t k0 = (int64_t)blockIdx.y * a.kc, k1 = k0 + a.kc < a.cols ? k0 + a.kc : a.cols;
  const int kn = (int)(k1 - k0);            // a multiple of 32
  const int xs = (int)a.kc + 8;             // LDS row stride (halves)
  {
    // eight of the thread's float4 of x in flight at a time (a loop of one load each waited for
    // every load in turn)
    const int q4 = kn / 4, tot = NBP * q4;
    for (int base = threadIdx.x; base < tot; base += 8 * NT) {
      float4v v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int idx = base + k * NT;
        const int b = idx / q4, q = idx - b * q4;
        v[k] = float4v{0.f, 0.f, 0.f, 0.f};
        if (idx < tot && b < a.B) v[k] = *reinterpret_cast<const float4v*>(a.x + (int64_t)b * a.cols + k0 + 4 * q);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int idx = base + k * NT;
        if (idx < tot) {
          const int b = idx / q4, q = idx - b * q4;
          half4_t h;
          h[0] = (_Float16)v[k][0]; h[1] = (_Float16)v[k][1]; h[2] = (_Float16)v[k][2]; h[3] = (_Float16)v[k][3];
          *reinterpret_cast<half4_t*>(xh + b * xs + 4 * q) = h;
          if constexpr (HILO) {
            half4_t l;
#pragma unroll
            for (int e = 0; e < 4; ++e) l[e] = (_Float16)(v[k][e] - (float)h[e]);
            *reinterpret_cast<half4_t*>(xh + (NBP + b) * xs + 4 * q) = l;
          }
        }
      }
    }
  }
  __syncthreads();
  const int tile = blockIdx.x * WPB + wave;
  if ((int64_t)tile * 16 >= count) return;
  const int g = lane / 16, ml = lane % 16;
  const int64_t pos = (int64_t)tile * 16 + ml;
  int64_t row = pos < count ? (a.list ? (int64_t)a.list[pos] : pos) : -1;
  if (row >= a.n_rows) row = -1;
  const int64_t rb = a.cols * 2;
  const uint32_t wbytes = (uint32_t)(a.n_rows * rb);
  const rsrc_t rW = make_rsrc(a.W, wbytes);
  const rsrc_t rU = make_rsrc(GATED ? a.Wup : a.W, GATED ? wbytes : 0u);
  const uint32_t roff = row >= 0 ? (uint32_t)(row * rb + (k0 + 8 * g) * 2) : 0u;
  constexpr uint32_t kOut = 0xFFFFFFF0u;
  float4v_t acc[NBT], accu[NBT];
#pragma unroll
  for (int t = 0; t < NBT; ++t) {
    acc[t] = float4v_t{0.f, 0.f, 0.f, 0.f};
    accu[t] = float4v_t{0.f, 0.f, 0.f, 0.f};
  }
  for (int kk = 0; kk < kn; kk += D * 32) {
    uint4 wv[D], uv[D];
#pragma unroll
    for (int i = 0; i < D; ++i) {
      const bool in = row >= 0 && kk + 32 * i < kn;
      const uint32_t o = in ? roff + (uint32_t)((kk + 32 * i) * 2) : kOut;
      wv[i] = bload16(rW, o);
      if constexpr (GATED) uv[i] = bload16(rU, o);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < D; ++i) {
      if (kk + 32 * i < kn) {
#pragma unroll
        for (int t = 0; t < NBT; ++t) {
          const half8_t xb = *reinterpret_cast<const half8_t*>(xh + (16 * t + ml) * xs + kk + 32 * i + 8 * g);
          acc[t] = mfma16(__builtin_bit_cast(half8_t, wv[i]), xb, acc[t]);
          if constexpr (GATED) accu[t] = mfma16(__builtin_bit_cast(half8_t, uv[i]), xb, accu[t]);
          if constexpr (HILO) {
            const half8_t xl =
                *reinterpret_cast<const half8_t*>(xh + (NBP + 16 * t + ml) * xs + kk + 32 * i + 8 * g);
            acc[t] = mfma16(__builtin_bit_cast(half8_t, wv[i]), xl, acc[t]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NBT; ++t) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t p = (int64_t)tile * 16 + 4 * g + r;
      if (p < count) {
        const int64_t o = ((int64_t)blockIdx.y * a.count_max + p) * NBP + 16 * t + ml;
        a.partials[o] = acc[t][r];
        if constexpr (GATED) a.partials[(int64_t)a.ks * a.count_max * NBP + o] = accu[t][r];
      }
    }
  }
}

// out[b * out_stride + pos] = finish(sum over ks of partials[ks][pos][b]) for pos < count, b < B.
template <bool GATED>
__global__ __launch_bounds__(256) void k_mm_finish(MmRowArgs a) {
  const int NBP = 16 * a.nbt;
  int64_t count = a.count_max;
  if (a.list) {
    const int64_t kd = *a.count_dev;
    count = kd < 0 ? 0 : (kd < a.count_max ? kd : a.count_max);
  }
  const int64_t n = count * NBP;
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < n; t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t pos = t / NBP;
    const int b = (int)(t % NBP);
    if (b >= a.B) continue;
    // partials loaded eight at a time (all in flight), summed in chunk order
    auto chunk_sum = [&](int half) {
      float acc = 0.f;
      for (int k0 = 0; k0 < a.ks; k0 += 8) {
        float p[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
          p[q] = k0 + q < a.ks ? a.partials[((int64_t)(half * a.ks + k0 + q) * a.count_max + pos) * NBP + b] : 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) acc += p[q];
      }
      return acc;
    };
    float z = chunk_sum(0), u = 0.f;
    if constexpr (GATED) u = chunk_sum(1);
    int64_t row = a.list ? (int64_t)a.list[pos] : pos;
    const bool ok = row >= 0 && row < a.n_rows;
    if (a.bias && ok) z += load_bias(a.bias, a.bias_dt, row);
    if (a.relu) z = z > 0.f ? z : 0.f;
    if constexpr (GATED) z *= u;
    a.out[(int64_t)b * a.out_stride + pos] = ok ? z : 0.f;
  }
}

// The same, written neuron-major: out[pos * NBP + b], zeros for b >= B.  NBP is a compile-time 16
// or 32, so the element's position and batch row are a shift and a mask; the indices fit 32 bits
// (PI_MAX_NEURONS positions x 32 batch rows x the split-K chunks of both products, under 2^31).
template <bool GATED, int NBT>
__global__ __launch_bounds__(256) void k_mm_finish_tr(MmRowArgs a) {
  constexpr int NBP = 16 * NBT;
  int count = (int)a.count_max;
  if (a.list) {
    const int64_t kd = *a.count_dev;
    count = kd < 0 ? 0 : (kd < a.count_max ? (int)kd : (int)a.count_max);
  }
  // the fp16 layout is written up to the next multiple of 32 positions (zeros), so
  // that the axpy's 8-position vectors never hold stale values.  Within each block of 32
  // positions, vector q (of four) holds positions q, q + 4, ..., q + 28: the rows that lane
  // group q of the axpy loads, in the order of its k slots
  const int npos = a.out_h8 ? (count + 31) / 32 * 32 : count;
  const int n = npos * NBP;
  const int cmax = (int)a.count_max;
  for (int t = blockIdx.x * blockDim.x + threadIdx.x; t < n; t += gridDim.x * blockDim.x) {
    const int pos = t / NBP;
    const int b = t % NBP;
    const int h8 = (((pos / 32) * 4 + pos % 4) * NBP + b) * 8 + (pos % 32) / 4;
    if (pos >= count) {
      reinterpret_cast<_Float16*>(a.out)[h8] = (_Float16)0.f;
      if (a.out_lo) reinterpret_cast<_Float16*>(a.out_lo)[h8] = (_Float16)0.f;
      continue;
    }
    float z = 0.f, u = 0.f;
    for (int k0 = 0; k0 < a.ks; k0 += 8) {
      float p[8], q[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p[i] = k0 + i < a.ks ? a.partials[((k0 + i) * cmax + pos) * NBP + b] : 0.f;
        if constexpr (GATED)
          q[i] = k0 + i < a.ks ? a.partials[((a.ks + k0 + i) * cmax + pos) * NBP + b] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        z += p[i];
        if constexpr (GATED) u += q[i];
      }
    }
    int64_t row = a.list ? (int64_t)a.list[pos] : pos;
    const bool ok = row >= 0 && row < a.n_rows && b < a.B;
    if (a.bias && ok) z += load_bias(a.bias, a.bias_dt, row);
    if (a.relu) z = z > 0.f ? z : 0.f;
    if constexpr (GATED) z *= u;
    if (a.out_h8) {
      const float v = ok ? z : 0.f;
      const _Float16 hi = (_Float16)v;
      reinterpret_cast<_Float16*>(a.out)[h8] = hi;
      if (a.out_lo) reinterpret_cast<_Float16*>(a.out_lo)[h8] = (_Float16)(v - (float)hi);
    } else {
      a.out[pos * NBP + b] = ok ? z : 0.f;
    }
  }
}

template <int DT, int NBT>
__global__ __launch_bounds__(kMmThreads) void k_mm_axpy(MmAxpyArgs a) {
  constexpr int E = Fmt<DT>::E;
  constexpr int D = 8;                      // row steps (4 rows each) in flight per wave
  __shared__ float red[kMmWaves][NBT * E * 4][kWave];
  extern __shared__ int32_t ax_rows[];     // the chunk's row ids (rows_per_chunk entries)
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int g = lane / 16, nl = lane % 16;
  const int cchunk = blockIdx.x, rchunk = blockIdx.y;
  int64_t count = a.count_max;
  if (a.list) {
    const int64_t kd = *a.count_dev;
    count = kd < 0 ? 0 : (kd < a.count_max ? kd : a.count_max);
  }
  const int64_t r0 = (int64_t)rchunk * a.rows_per_chunk;
  int64_t r1 = r0 + a.rows_per_chunk;
  r1 = r1 < count ? r1 : count;
  // row ids of the chunk, looked up once (listed rows) so that no weight load
  // waits on a list load inside the loop
  for (int64_t j = r0 + threadIdx.x; j < r1; j += kMmThreads) {
    int64_t row = a.list ? (int64_t)a.list[j] : j;
    ax_rows[j - r0] = (row >= 0 && row < a.n_rows) ? (int32_t)row : -1;
  }
  __syncthreads();
  const int64_t rb = row_bytes(DT, a.cols);
  const int64_t groups = a.cols / 128;
  const int nvec = (int)(rb / 16);
  const int v = cchunk * 16 + nl;           // this lane's 16-byte vector of each row
  const bool vin = v < nvec;
  const uint32_t wbytes = (uint32_t)(a.n_rows * rb);
  const rsrc_t rW = make_rsrc(a.W, wbytes);
  const rsrc_t rS = make_rsrc(DT == 2 ? (const void*)a.Ws : a.W, DT == 2 ? (uint32_t)(a.n_rows * groups * 2) : 0u);
  const int NBP = 16 * NBT;
  const rsrc_t rA = make_rsrc(a.a, a.a_tr ? (uint32_t)((a.a_by_row ? a.n_rows : a.count_max) * NBP * 4)
                                          : (uint32_t)(a.B * a.a_stride * 4));
  float4v_t acc[NBT][E];
#pragma unroll
  for (int t = 0; t < NBT; ++t)
#pragma unroll
    for (int e = 0; e < E; ++e) acc[t][e] = float4v_t{0.f, 0.f, 0.f, 0.f};
  // row steps of 4 rows: step st covers rows r0 + 4 st .. +3, wave st % 4.  A round
  // is D steps of one wave, all its loads issued before its instructions.  (Issuing
  // round i+1 before computing round i needs twice the registers, and the
  // occupancy lost costs more than the overlap gains.)
  struct Round {
    uint4 wv[D];
    float sc[D], av[D][NBT];
  };
  constexpr int64_t kStep = 4 * kMmWaves * D;
  auto issue = [&](int64_t j0, Round& rd) {
    int32_t rowv[D];
#pragma unroll
    for (int i = 0; i < D; ++i) {                 // every row id of the round first (one LDS wait)
      const int64_t j = j0 + (int64_t)4 * kMmWaves * i + g;
      rowv[i] = j < r1 ? ax_rows[j - r0] : -1;
    }
#pragma unroll
    for (int i = 0; i < D; ++i) {
      const int64_t j = j0 + (int64_t)4 * kMmWaves * i + g;
      const int64_t row = rowv[i];
      const bool ok = row >= 0 && vin;
      rd.wv[i] = bload16(rW, ok ? (uint32_t)(row * rb) + (uint32_t)v * 16u : 0xFFFFFFF0u);
      if constexpr (DT == 2) rd.sc[i] = h2f(bload2(rS, ok ? (uint32_t)(row * groups + v / 4) * 2u : 0xFFFFFFF0u));
      const int64_t ai = a.a_by_row ? (row >= 0 ? row : 0) : j;
#pragma unroll
      for (int t = 0; t < NBT; ++t) {
        const int b = 16 * t + nl;
        // neuron-major activations: the 16 lanes of a row group read 64 contiguous bytes
        const uint32_t off = a.a_tr ? (uint32_t)((ai * NBP + b) * 4) : (uint32_t)((b * a.a_stride + ai) * 4);
        rd.av[i][t] = __uint_as_float(
            __builtin_amdgcn_raw_buffer_load_b32(rA, (row >= 0 && b < a.B) ? (int)off : -16, 0, 0));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto compute = [&](const Round& rd) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      float wf[E];
      widen_vec<DT>(rd.wv[i], DT == 2 ? rd.sc[i] : 1.f, wf);
      // A[m = b][k = row g] = a[b][row], B[k = row g][n] = W[row][column of tile e]
#pragma unroll
      for (int e = 0; e < E; ++e)
#pragma unroll
        for (int t = 0; t < NBT; ++t) acc[t][e] = mfma4(rd.av[i][t], wf[e], acc[t][e]);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int64_t j0 = r0 + 4 * wave; j0 < r1; j0 += kStep) {
    Round rd;
    issue(j0, rd);
    compute(rd);
  }
  // sum the four waves in wave order; lane holds D[m = 4g + r][n = lane % 16] of each tile
#pragma unroll
  for (int t = 0; t < NBT; ++t)
#pragma unroll
    for (int e = 0; e < E; ++e)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][(t * E + e) * 4 + r][lane] = acc[t][e][r];
  __syncthreads();
  const int64_t cols = a.cols;
  for (int q = threadIdx.x; q < NBT * E * 4 * kWave; q += kMmThreads) {
    const int ln = q % kWave, idx = q / kWave;
    const int r = idx % 4, te = idx / 4, e = te % E, t = te / E;
    const int b = 16 * t + 4 * (ln / 16) + r;
    const int64_t c = (int64_t)(cchunk * 16 + (ln % 16)) * E + e;
    if (b < a.B && c < cols) {
      float s = red[0][idx][ln];
#pragma unroll
      for (int w = 1; w < kMmWaves; ++w) s += red[w][idx][ln];
      a.partials[((int64_t)rchunk * a.B + b) * cols + c] = s;
    }
  }
}

// fp16 weights, fp16 activations (FC2 of the batched path): one
// v_mfma_f32_16x16x32_f16 sums 32 listed rows.  Lane (g = lane / 16, n = lane % 16)
// of a row step loads rows js + 4 i + g (i = 0 .. 7), each row's 16-byte vector n of
// the block's 128 columns: 8 rows x 8 columns in its own registers.  Those rows are
// its k slots 8 g .. 8 g + 7, so instruction s2 takes half s2 of each row vector as
// B (column 8 n + s2; a transpose in registers, no LDS), and A = a for batch row
// lane % 16 at the same 8 rows, one 16-byte vector of the fp16 activation layout
// (which stores positions q, q + 4, .., q + 28 of each 32-block in vector q).  The
// block's WV waves take interleaved row steps and
// are summed in LDS in wave order.  With LO, a = hi + lo in two fp16 parts
// (about 22 bits): two exact products per weight, for the predictor's output
// layer, whose logits keep near-fp32 precision.  That layer is one row chunk
// over all H rows with one block per 128 columns (fewer blocks than compute
// units at these sizes), so it takes eight waves per block: half the rounds of
// dependent loads per wave.  FC2 keeps four, with several blocks per unit.
__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

template <int NBT, bool LO, int WV>
__global__ __launch_bounds__(WV * kWave) void k_mm_axpy16(MmAxpyArgs a) {
  constexpr int DS = 2;                     // row steps in flight per wave
  constexpr int kThreads = WV * kWave;
  __shared__ float red[NBT * 8 * 4][kWave + 1];
  extern __shared__ int32_t ax_rows[];     // the chunk's row ids (rows_per_chunk entries)
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int g = lane / 16, nl = lane % 16;
  const int cchunk = blockIdx.x, rchunk = blockIdx.y;
  int64_t count = a.count_max;
  if (a.list) {
    const int64_t kd = *a.count_dev;
    count = kd < 0 ? 0 : (kd < a.count_max ? kd : a.count_max);
  }
  // the row chunks split the device count evenly (multiples of 32 rows; no more than the
  // rows_per_chunk the LDS row ids are sized for, which bounds count_max / row_chunks)
  int64_t rpc = ((count + a.row_chunks - 1) / a.row_chunks + 31) / 32 * 32;
  rpc = rpc < a.rows_per_chunk ? rpc : a.rows_per_chunk;
  const int64_t r0 = (int64_t)rchunk * rpc;
  int64_t r1 = r0 + rpc;
  r1 = r1 < count ? r1 : count;
  for (int64_t j = r0 + threadIdx.x; j < r1; j += kThreads) {
    const int64_t row = a.list ? (int64_t)a.list[j] : j;
    ax_rows[j - r0] = (row >= 0 && row < a.n_rows) ? (int32_t)row : -1;
  }
  __syncthreads();
  // with the logits written here, thread cc < 128 adds the output bias of column 128 cchunk + cc:
  // loaded now, so it is not a round trip after the sums
  const float cb_early = (a.final_out && a.bias && threadIdx.x < 128 && (int64_t)cchunk * 128 + threadIdx.x < a.cols)
                             ? load_bias(a.bias, a.bias_dt, (int64_t)cchunk * 128 + threadIdx.x) : 0.f;
  const int NBP = 16 * NBT;
  const int64_t rb = a.cols * 2;
  const int nvec = (int)(rb / 16);
  const int v = cchunk * 16 + nl;           // this lane's 16-byte chunk of each row it loads
  const bool vin = v < nvec;
  const rsrc_t rW = make_rsrc(a.W, (uint32_t)(a.n_rows * rb));
  const uint32_t abytes = (uint32_t)((a.count_max + 31) / 32 * 32 * NBP * 2);
  const rsrc_t rA = make_rsrc(a.a, abytes);
  const rsrc_t rL = make_rsrc(LO ? (const void*)a.a_lo : (const void*)a.a, LO ? abytes : 0u);
  constexpr uint32_t kOut = 0xFFFFFFF0u;
  float4v_t acc[NBT][8];
#pragma unroll
  for (int t = 0; t < NBT; ++t)
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) acc[t][s2] = float4v_t{0.f, 0.f, 0.f, 0.f};
  constexpr int kBlockStep = 32 * WV;
  for (int64_t j0 = r0 + 32 * wave; j0 < r1; j0 += (int64_t)kBlockStep * DS) {
    uint4 wv[DS][8], av[DS][NBT], al[DS][NBT];
#pragma unroll
    for (int st = 0; st < DS; ++st) {
      const int64_t js = j0 + (int64_t)kBlockStep * st;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t j = js + 4 * i + g;
        const int32_t row = j < r1 ? ax_rows[j - r0] : -1;
        wv[st][i] = bload16(rW, row >= 0 && vin ? (uint32_t)(row * rb) + (uint32_t)v * 16u : kOut);
      }
#pragma unroll
      for (int t = 0; t < NBT; ++t) {
        // the lane's k slots are rows js + 4 i + g: vector g of the 32-position block at js
        const uint32_t ao = js < r1 ? (uint32_t)((((js / 32) * 4 + g) * NBP + 16 * t + nl) * 16) : kOut;
        av[st][t] = bload16(rA, ao);
        if constexpr (LO) al[st][t] = bload16(rL, ao);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 0; st < DS; ++st) {
      if (j0 + (int64_t)kBlockStep * st < r1) {
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) {
          // the lane's 8 rows (k slots 8 g .. 8 g + 7) hold its columns 8 nl .. 8 nl + 7:
          // instruction s2 takes column 8 nl + s2, half s2 of each row vector (a transpose in
          // registers; output column n = nl of instruction s2 is column 8 nl + s2)
          uint32_t wb[4];
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const uint32_t lo = word_of(wv[st][2 * p], s2 / 2), hi = word_of(wv[st][2 * p + 1], s2 / 2);
            wb[p] = (s2 & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
          }
          const half8_t wh = __builtin_bit_cast(half8_t, uint4{wb[0], wb[1], wb[2], wb[3]});
#pragma unroll
          for (int t = 0; t < NBT; ++t) {
            acc[t][s2] = mfma16(__builtin_bit_cast(half8_t, av[st][t]), wh, acc[t][s2]);
            if constexpr (LO) acc[t][s2] = mfma16(__builtin_bit_cast(half8_t, al[st][t]), wh, acc[t][s2]);
          }
        }
      }
    }
  }
  // sum the four waves in wave order; lane holds D[m = 4g + r][n = nl] of each (t, s2)
  for (int w = 0; w < WV; ++w) {
    if (wave == w) {
#pragma unroll
      for (int t = 0; t < NBT; ++t)
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float* cell = &red[(t * 8 + s2) * 4 + r][lane];
            *cell = w == 0 ? acc[t][s2][r] : *cell + acc[t][s2][r];
          }
    }
    __syncthreads();
  }
  const int64_t cols = a.cols;
  if (a.final_out) {
    // one row chunk: the whole sum is here.  Thread cc of the block's first two
    // waves takes column c0 + cc over every batch row, so each wave's ballot is
    // the union word of one 64-column group.
    if (threadIdx.x < 128) {
      const int cc = threadIdx.x, s2 = cc % 8, n = cc / 8;   // column 8 n + s2 of the tile
      const int64_t c = (int64_t)cchunk * 128 + cc;
      const bool cin = c < cols;
      const float cb = cb_early;
      bool f = false;
      for (int b = 0; b < a.B; ++b) {
        const int t = b / 16, g2 = (b % 16) / 4, r = b % 4;
        float z = 0.f + red[(t * 8 + s2) * 4 + r][16 * g2 + n];
        if (a.bias) z += cb;
        if (cin) a.final_out[(int64_t)b * cols + c] = z;
        f = f || (cin && z > a.tau);
      }
      const uint64_t M = __ballot(f);
      const int64_t grp = (int64_t)cchunk * 2 + threadIdx.x / kWave;
      if (a.mask && (threadIdx.x & (kWave - 1)) == 0 && grp * 64 < cols) {
        a.mask[2 * grp] = (uint32_t)M;
        a.mask[2 * grp + 1] = (uint32_t)(M >> 32);
      }
    }
    return;
  }
  // thread q: column 8 n + s2 of the tile (consecutive threads, consecutive columns), batch row
  // 16 t + 4 g + r
  for (int q = threadIdx.x; q < NBT * 8 * 4 * kWave; q += kThreads) {
    const int s2 = q % 8, n = (q / 8) % 16, r = (q / 128) % 4, g2 = (q / 512) % 4, t = q / 2048;
    const int b = 16 * t + 4 * g2 + r;
    const int64_t c = (int64_t)cchunk * 128 + 8 * n + s2;
    if (b < a.B && c < cols) a.partials[((int64_t)rchunk * a.B + b) * cols + c] = red[(t * 8 + s2) * 4 + r][16 * g2 + n];
  }
}

template <int DT>
hipError_t rowdot_dt(const MmRowArgs& a, hipStream_t s) {
  const int tiles = (int)((a.count_max + 15) / 16);
  const dim3 g((unsigned)((tiles + kMmWaves - 1) / kMmWaves), (unsigned)a.ks), t(kMmThreads);
  if (mm_row16_used(a)) {
    const size_t shm = (size_t)16 * a.nbt * (size_t)(a.kc + 8) * 2 * (a.x_hilo ? 2 : 1);
    const int wpb = r16_waves(a.nbt);
    const dim3 g((unsigned)((tiles + wpb - 1) / wpb), (unsigned)a.ks), t(wpb * kWave);
    if (a.x_hilo) {          // the predictor's hidden layer: never gated
      if (a.nbt == 1) hipLaunchKernelGGL((k_mm_rowdot16<1, false, true>), g, t, shm, s, a);
      else hipLaunchKernelGGL((k_mm_rowdot16<2, false, true>), g, t, shm, s, a);
    } else if (a.nbt == 1) {
      if (a.gated) hipLaunchKernelGGL((k_mm_rowdot16<1, true, false>), g, t, shm, s, a);
      else hipLaunchKernelGGL((k_mm_rowdot16<1, false, false>), g, t, shm, s, a);
    } else {
      if (a.gated) hipLaunchKernelGGL((k_mm_rowdot16<2, true, false>), g, t, shm, s, a);
      else hipLaunchKernelGGL((k_mm_rowdot16<2, false, false>), g, t, shm, s, a);
    }
    return hipGetLastError();
  }
  if (a.nbt == 1) {
    if (a.gated) hipLaunchKernelGGL((k_mm_rowdot<DT, 1, true>), g, t, 0, s, a);
    else hipLaunchKernelGGL((k_mm_rowdot<DT, 1, false>), g, t, 0, s, a);
  } else {
    if (a.gated) hipLaunchKernelGGL((k_mm_rowdot<DT, 2, true>), g, t, 0, s, a);
    else hipLaunchKernelGGL((k_mm_rowdot<DT, 2, false>), g, t, 0, s, a);
  }
  return hipGetLastError();
}

template <int DT>
hipError_t axpy_dt(const MmAxpyArgs& a, hipStream_t s) {
  const dim3 g((unsigned)mm_axpy_col_chunks(a.dt, a.cols), (unsigned)a.row_chunks), t(kMmThreads);
  const size_t shm = (size_t)a.rows_per_chunk * 4;
  if (DT == 1 && a.a_h8) {
    if (a.a_lo && a.final_out && a.rows_per_chunk <= kOutWavesMaxRows) {
      const dim3 t8(kOutWaves * kWave);
      if (a.nbt == 1) hipLaunchKernelGGL((k_mm_axpy16<1, true, kOutWaves>), g, t8, shm, s, a);
      else hipLaunchKernelGGL((k_mm_axpy16<2, true, kOutWaves>), g, t8, shm, s, a);
    } else if (a.a_lo) {
      if (a.nbt == 1) hipLaunchKernelGGL((k_mm_axpy16<1, true, kMmWaves>), g, t, shm, s, a);
      else hipLaunchKernelGGL((k_mm_axpy16<2, true, kMmWaves>), g, t, shm, s, a);
    } else {
      if (a.nbt == 1) hipLaunchKernelGGL((k_mm_axpy16<1, false, kMmWaves>), g, t, shm, s, a);
      else hipLaunchKernelGGL((k_mm_axpy16<2, false, kMmWaves>), g, t, shm, s, a);
    }
    return hipGetLastError();
  }
  if (a.nbt == 1) hipLaunchKernelGGL((k_mm_axpy<DT, 1>), g, t, shm, s, a);
  else hipLaunchKernelGGL((k_mm_axpy<DT, 2>), g, t, shm, s, a);
  return hipGetLastError();
}

}  // namespace

int mm_nbt(int B) { return B <= 16 ? 1 : 2; }

int mm_row_ks(int dt, int64_t count_max, int64_t cols) {
  // about 2048 waves, each over at least 8 k blocks
  const int64_t kb = 4 * (dt == 0 ? 4 : dt == 1 ? 8 : 32);
  const int64_t tiles = (count_max + 15) / 16;
  int64_t ks = (2048 + tiles - 1) / (tiles > 0 ? tiles : 1);
  const int64_t kmax = cols / (8 * kb);
  ks = ks > kmax ? kmax : ks;
  return (int)(ks < 1 ? 1 : ks);
}

bool mm_row16_used(const MmRowArgs& a) {
  if (a.x_hilo && a.gated) return false;
  return (a.x_f16 || a.x_hilo) && a.dt == PI_F16 && a.cols % 32 == 0 && a.kc <= row16_kcmax(a.nbt, a.x_hilo) &&
         a.kc % 32 == 0;
}

int mm_row16_ks(int64_t count_max, int64_t cols, int nbt, bool gated, bool hilo) {
  // the k chunk fits the LDS bound, and about 4096 waves
  (void)gated;
  const int64_t kcmax = row16_kcmax(nbt, hilo);
  const int64_t tiles = (count_max + 15) / 16;
  int64_t ks = (4096 + tiles - 1) / (tiles > 0 ? tiles : 1);
  const int64_t kmax = cols / 256;          // at least 8 k blocks per wave
  ks = ks > kmax ? kmax : ks;
  const int64_t kmin = (cols + kcmax - 1) / kcmax;
  ks = ks < kmin ? kmin : ks;
  return (int)(ks < 1 ? 1 : ks);
}

int64_t mm_row_kc(int dt, int64_t cols, int ks) {
  const int64_t kb = 4 * (dt == 0 ? 4 : dt == 1 ? 8 : 32);
  const int64_t blocks = (cols + kb - 1) / kb;
  return ((blocks + ks - 1) / ks) * kb;
}

int mm_axpy_col_chunks(int dt, int64_t cols) {
  const int64_t nvec = row_bytes(dt, cols) / 16;
  return (int)((nvec + 15) / 16);
}

int mm_axpy_row_chunks(int dt, int nbt, int64_t count_max, int64_t cols) {
  // fp16: one resident round of blocks (3 per CU for 16 batch rows, 2 for 32, set by
  // the registers); others: about 1024 blocks of four waves
  const int64_t cc = mm_axpy_col_chunks(dt, cols);
  const int64_t target = dt == PI_F16 ? (int64_t)(nbt == 1 ? 3 : 2) * kNumCU : 1024;
  int64_t rc = dt == PI_F16 ? target / cc : (target + cc - 1) / cc;
  const int64_t rmax = (count_max + 63) / 64;   // at least 64 rows per block
  rc = rc > rmax ? rmax : rc;
  return (int)(rc < 1 ? 1 : rc);
}

bool mm_rowdot_supported(int dt, int64_t rows, int64_t cols) {
  if (dt < 0 || dt > 2) return false;
  const int64_t kb = 4 * (dt == 0 ? 4 : dt == 1 ? 8 : 32);
  return cols % kb == 0 && rows * row_bytes(dt, cols) < ((int64_t)1 << 31);
}

bool mm_axpy16_supported(int dt, int64_t cols) { return dt == PI_F16 && cols % 8 == 0; }

int64_t mm_axpy_rows_per_chunk(const MmAxpyArgs& a) {
  // a multiple of 16 rows (128 for the fp16 kernel, whose block step is 128 rows)
  const int64_t q = a.a_h8 ? 128 : 16;
  return ((a.count_max + a.row_chunks - 1) / a.row_chunks + q - 1) / q * q;
}

bool mm_axpy_supported(int dt, int64_t rows, int64_t cols) {
  // int4 rows would give 32 column tiles per lane vector: the VALU axpy takes them
  return (dt == 0 || dt == 1) && rows * row_bytes(dt, cols) < ((int64_t)1 << 31);
}

hipError_t launch_mm_rowdot(const MmRowArgs& a, hipStream_t s) {
  hipError_t e;
  switch (a.dt) {
    case 0: e = rowdot_dt<0>(a, s); break;
    case 1: e = rowdot_dt<1>(a, s); break;
    default: e = rowdot_dt<2>(a, s); break;
  }
  if (e != hipSuccess) return e;
  const int64_t n = a.count_max * 16 * a.nbt;
  int64_t blocks = (n + 255) / 256;
  blocks = blocks < 1 ? 1 : (blocks > 2048 ? 2048 : blocks);
  if (a.out_tr) {
    if (a.nbt == 1) {
      if (a.gated) hipLaunchKernelGGL((k_mm_finish_tr<true, 1>), dim3((unsigned)blocks), dim3(256), 0, s, a);
      else hipLaunchKernelGGL((k_mm_finish_tr<false, 1>), dim3((unsigned)blocks), dim3(256), 0, s, a);
    } else {
      if (a.gated) hipLaunchKernelGGL((k_mm_finish_tr<true, 2>), dim3((unsigned)blocks), dim3(256), 0, s, a);
      else hipLaunchKernelGGL((k_mm_finish_tr<false, 2>), dim3((unsigned)blocks), dim3(256), 0, s, a);
    }
  } else {
    if (a.gated) hipLaunchKernelGGL(k_mm_finish<true>, dim3((unsigned)blocks), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(k_mm_finish<false>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_mm_axpy(const MmAxpyArgs& a, hipStream_t s) {
  switch (a.dt) {
    case 0: return axpy_dt<0>(a, s);
    case 1: return axpy_dt<1>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pi
