// moe_mx.hip -- MI355X (gfx950) routed-experts MoE decode step: MXFP8 activations x
// FP4 (e2m1 + E8M0) expert weights, behind the C ABI of include/moe_mx.h.
//
// Sources (vLLM API documentation pages):
//   [experts]  "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.moe.experts"
//   [runtime]  "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.moe.experts_runtime"
// The pages' engine (TMA producer warp, TMEM accumulators, mbarriers, clusters) is
// NVIDIA-specific; this file keeps the method (MXFP8 plan, (expert, <=8 token) units,
// FC1 -> gated activation -> hidden requant -> FC2, rows in top-k order, contiguous
// work slices) and maps it onto CDNA4:
//   * weights stream from HBM once per distinct expert per call, through per-wave LDS
//     DMA rings (global_load_lds, 16 bytes per lane), as the operands of
//     v_mfma_scale_f32_16x16x128_f8f6f4 (FP4 A operand = a 16-row weight tile, FP8 B
//     operand = 16 token columns); block scales go to the MFMA as E8M0 operands;
//   * one persistent, co-resident kernel: every workgroup takes a contiguous slice of
//     the FC1 work, then of the FC2 work; four streaming waves per workgroup only
//     stream and multiply, one control wave does every cross-workgroup step;
//   * the FC1 -> FC2 hidden exchange and the split-block FC1 partial sums cross XCDs
//     through device-coherent (sc1) stores and loads, call-tagged flags and
//     agent-scope counters;
//   * for B <= 8 the step is one launch that also routes the batch and quantizes x (the
//     decode form): by default decode_whole_kernel, where each hidden block's FC1 runs
//     over the whole of K inside one workgroup and only the finished MXFP8 hidden
//     crosses workgroups, as call-tagged words; or the experts kernel's decode form.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>

#include "moe_mx.h"

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

constexpr int kStream = 4;        // streaming waves per experts workgroup
constexpr int kWG = 64 * (kStream + 1);  // plus one control wave
constexpr int kGroupThreads = 1024;
// Bounds of the waits on other waves' progress: far beyond any legitimate wait (a launch
// lasts well under a millisecond), short enough that a broken invariant ends the launch
// within tens of milliseconds.
constexpr uint32_t kSpinLimit = 1u << 19;  // polls of an LDS word (~40 ms)
constexpr uint32_t kPollLimit = 1u << 16;  // polls of a global flag (15-60 ms)

// ------------------------------------------------------------------ formats
// E8M0 exponent of an MX block from its absolute maximum (experts page, mx_block and
// store_hidden call mx_exponent).  Default rule: the smallest e with amax*2^-e <= 448;
// floor rule (OCP MX): e = floor(log2 amax) - 8.  amax == 0 -> -127.  Clamped to
// [-127, 127].
__device__ __forceinline__ int mx_exponent(float amax, bool floor_rule) {
  const uint32_t b = __float_as_uint(amax) & 0x7fffffffu;
  if (b == 0) return -127;
  int e = static_cast<int>(b >> 23) - 127 - 8;
  if (!floor_rule && (b & 0x7fffffu) > 0x600000u) e += 1;  // mantissa > 1.75
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// 2^-e as a binary32 (e in [-127, 126]: always a normal number).
__device__ __forceinline__ float exp2_neg(int e) {
  return __uint_as_float(static_cast<uint32_t>(127 - e) << 23);
}

// binary32 -> e4m3 (fn) code, round to nearest even, saturating to +-448.
__device__ __forceinline__ uint32_t to_e4m3(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a >= 0x43e00000u) return sign | 0x7eu;              // |v| >= 448
  if (a < 0x3c800000u) {                                    // |v| < 2^-6: step 2^-9
    const float m = __builtin_rintf(__uint_as_float(a) * 512.0f);
    return sign | static_cast<uint32_t>(m);                 // m == 8 encodes 2^-6
  }
  const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);       // RNE to 3 mantissa bits
  const uint32_t code = ((((r >> 23) - 120u) << 3) | ((r >> 20) & 7u));
  return sign | (code > 0x7eu ? 0x7eu : code);
}

__device__ __forceinline__ uint32_t to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// ------------------------------------------------------ coherent accesses
// Data handed between workgroups of one launch may sit in different XCDs' L2s; these
// agent-scope relaxed atomics are device-coherent (sc1) and are ordered by an explicit
// vmcnt wait before the flag that publishes them.
__device__ __forceinline__ uint32_t ld_dev_u32(const void* p) {
  return __hip_atomic_load(reinterpret_cast<const uint32_t*>(p), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev_u64(const void* p) {
  return __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev_u32(void* p, uint32_t v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev_u64(void* p, uint64_t v) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Give-up test of a bounded wait on flags in global memory: true after kPollLimit polls
// (tens of milliseconds), or, checked every 256 polls, once any wave of the launch has
// given up and set bit 2 of the status word, so that one broken wait ends the others
// within about a millisecond instead of each running out its own bound.
__device__ __forceinline__ bool poll_expired(uint32_t spins, const int32_t* err) {
  return (spins & 255u) == 255u && (spins >= kPollLimit || (ld_dev_u32(err) & 4u) != 0);
}
__device__ __forceinline__ void st_dev_u8(void* p, uint8_t v) {
  __hip_atomic_store(reinterpret_cast<uint8_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ uint4 ld16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint32_t ld4(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }

__device__ __forceinline__ v8i fp4_operand(uint4 a) {
  v8i r = {static_cast<int>(a.x), static_cast<int>(a.y), static_cast<int>(a.z), static_cast<int>(a.w),
           0, 0, 0, 0};
  return r;
}
// Block-scaled FP4 (A, 16 rows) x FP8 (B, 16 columns) -> FP32 16x16 tile, K = 128.
// The destination of this multi-pass MFMA must not share registers with A or B (it is
// written while they are still read); in its VGPR-destination form the compiler does not
// enforce that, so kernels that use it declare AGPR use (agpr_form()) and the compiler
// gives the MFMA accumulation registers of their own.
__device__ __forceinline__ v4f mfma_fp4_fp8(v8i a, v8i b, v4f c, int scale_a, int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 0, 0, scale_a, 0, scale_b);
}
__device__ __forceinline__ void agpr_form() { asm volatile("" : : : "a0"); }
// Extra wait states before results of the MFMA above are read by ordinary instructions:
// the compiler's count is short for this FP4 x FP8 K = 128 form (the first result
// register is ready, the later ones are not).  The accumulators are asm operands, so
// no read of them can move ahead of the wait.
__device__ __forceinline__ void mfma_settle(v4f& x) { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(x)); }
__device__ __forceinline__ void mfma_settle(v4f& x0, v4f& x1, v4f& x2, v4f& x3) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(x0), "+a"(x1), "+a"(x2), "+a"(x3));
}
__device__ __forceinline__ v8i fp8_operand(uint4 lo, uint4 hi) {
  v8i r = {static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z), static_cast<int>(lo.w),
           static_cast<int>(hi.x), static_cast<int>(hi.y), static_cast<int>(hi.z), static_cast<int>(hi.w)};
  return r;
}

// ------------------------------------------------------------------ plan
// MXFP8 quantization of x (experts page, plan_chunk: the same quantization as mx_block),
// four lanes per 32-element block of a token row: one 16-byte load and one 8-byte store
// each, the block's amax combined across the four lanes.  x: BF16 [B, D]; codes [B, D];
// scales [B, D/32]; idx4 = 4 * block + quarter.
__device__ __forceinline__ void plan_quarter(const uint8_t* __restrict__ x, int64_t idx4, uint8_t* __restrict__ codes,
                                             uint8_t* __restrict__ scales) {
  const uint4 q = ld16(x + idx4 * 16);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  float v[8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    amax = fmaxf(amax, fmaxf(fabsf(v[2 * i]), fabsf(v[2 * i + 1])));
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  const int e = mx_exponent(amax, false);
  const float sc = exp2_neg(e);
  uint32_t c[2];
#pragma unroll
  for (int k = 0; k < 2; ++k)
    c[k] = to_e4m3(v[4 * k] * sc) | (to_e4m3(v[4 * k + 1] * sc) << 8) | (to_e4m3(v[4 * k + 2] * sc) << 16) |
           (to_e4m3(v[4 * k + 3] * sc) << 24);
  *reinterpret_cast<uint2*>(codes + idx4 * 8) = make_uint2(c[0], c[1]);
  if ((idx4 & 3) == 0) scales[idx4 >> 2] = static_cast<uint8_t>(e + 127);
}

// plan_quarter with device-coherent stores (sc1: written through to memory, so that other
// workgroups of the same launch read them after an acquire; no L2 write-back needed).
// From the quarter's 16 bytes of x, already loaded.
__device__ __forceinline__ void plan_quarter_dev_v(const uint4 q, int64_t idx4, uint8_t* __restrict__ codes,
                                                   uint8_t* __restrict__ scales) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  float v[8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    amax = fmaxf(amax, fmaxf(fabsf(v[2 * i]), fabsf(v[2 * i + 1])));
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  const int e = mx_exponent(amax, false);
  const float sc = exp2_neg(e);
  uint32_t c[2];
#pragma unroll
  for (int k = 0; k < 2; ++k)
    c[k] = to_e4m3(v[4 * k] * sc) | (to_e4m3(v[4 * k + 1] * sc) << 8) | (to_e4m3(v[4 * k + 2] * sc) << 16) |
           (to_e4m3(v[4 * k + 3] * sc) << 24);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(codes + idx4 * 8), static_cast<uint64_t>(c[0]) | (static_cast<uint64_t>(c[1]) << 32),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if ((idx4 & 3) == 0)
    __hip_atomic_store(scales + (idx4 >> 2), static_cast<uint8_t>(e + 127), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void plan_quarter_dev(const uint8_t* __restrict__ x, int64_t idx4, uint8_t* __restrict__ codes,
                                                 uint8_t* __restrict__ scales) {
  plan_quarter_dev_v(ld16(x + idx4 * 16), idx4, codes, scales);
}

__global__ __launch_bounds__(256) void plan_kernel(const uint8_t* __restrict__ x, int64_t nblocks,
                                                   uint8_t* __restrict__ codes,
                                                   uint8_t* __restrict__ scales) {
  const int64_t idx4 = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx4 < 4 * nblocks) plan_quarter(x, idx4, codes, scales);
}

// ------------------------------------------------------------------ combine
// Weighted top-k combine (experts page, ExpertsKernel.finalize without the multicast):
// out[t, d] = sum over s of w[t, s] * y[t*K + s, d], FP32 fused multiply-adds in slot
// order, rounded once to BF16.  One thread per 8 consecutive d of one token (16-byte
// row reads and one 16-byte store).
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ rows, const float* __restrict__ w,
                                                      int B, int K, int D, uint16_t* __restrict__ out) {
  const int per = D / 8;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<int64_t>(B) * per) return;
  const int t = static_cast<int>(i / per), c = static_cast<int>(i - static_cast<int64_t>(t) * per);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const uint16_t* r = rows + static_cast<int64_t>(t) * K * D + c * 8;
  for (int s = 0; s < K; ++s) {
    const float ws = w[static_cast<int64_t>(t) * K + s];
    const uint4 v = *reinterpret_cast<const uint4*>(r + static_cast<int64_t>(s) * D);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] = fmaf(ws, __uint_as_float(u[q] << 16), acc[2 * q]);
      acc[2 * q + 1] = fmaf(ws, __uint_as_float(u[q] & 0xffff0000u), acc[2 * q + 1]);
    }
  }
  uint32_t o[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) o[q] = to_bf16_bits(acc[2 * q]) | (to_bf16_bits(acc[2 * q + 1]) << 16);
  *reinterpret_cast<uint4*>(out + static_cast<int64_t>(t) * D + c * 8) = make_uint4(o[0], o[1], o[2], o[3]);
}

// ------------------------------------------------------------------ units buffer
// The unit table lives in its own caller buffer: header, per-unit expert and eight
// pair indices, then the distinct experts ("groups") with their first unit, unit count
// and first 16-column tile.
struct Table {
  int32_t* hdr;          // [16]: n_units, n_groups, n_tiles, flags (1: id out of range,
                         //        2: id repeated in a token, 4: a hidden wait timed out),
                         //        n_chunks
  int32_t* unit_expert;  // [U]
  int32_t* unit_rows;    // [U, 8]
  int32_t* g_expert;     // [G]
  int32_t* g_unit0;      // [G]
  int32_t* g_nunits;     // [G]
  int32_t* g_tile0;      // [G]
  // chunks of the grouped kernel: each expert's routes, in token order, cut into runs of
  // kChunkCols token columns (one weight pass of that expert each)
  int32_t* c_expert;     // [C]
  int32_t* c_cols;       // [C] real columns of the chunks before | real columns (1..kChunkCols) << 20
                         // (hdr[5]: the real columns of all chunks)
  int32_t* c_pairs;      // [C, kChunkCols] pair indices t*K + s, -1 where padded
};
constexpr int kChunkCols = 32;  // token columns per chunk: two 16-column MFMA tiles

constexpr size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

struct UnitsLayout {
  size_t hdr, unit_expert, unit_rows, g_expert, g_unit0, g_nunits, g_tile0, c_expert, c_cols, c_pairs, end;
  int64_t max_chunks;
};

// Chunks of a batch of U routes over at most G experts: sum_g ceil(n_g / 32) with
// sum_g n_g = U.
int64_t max_chunks_for(int64_t U, int64_t G) { return G + (U + kChunkCols - 1) / kChunkCols; }

UnitsLayout units_layout(int B, int K, int E) {
  UnitsLayout L{};
  const int64_t U = static_cast<int64_t>(B) * K;
  const int64_t G = U < E ? U : E;
  L.max_chunks = max_chunks_for(U, G);
  size_t off = 0;
  L.hdr = off;
  off += 64;
  L.unit_expert = off;
  off = align256(off + U * 4);
  L.unit_rows = off;  // 16-byte aligned: read as int4
  off += U * 32;
  L.g_expert = off;
  off += G * 4;
  L.g_unit0 = off;
  off += G * 4;
  L.g_nunits = off;
  off += G * 4;
  L.g_tile0 = off;
  off += G * 4;
  L.c_expert = align256(off);
  off = L.c_expert + L.max_chunks * 4;
  L.c_cols = off;
  off += L.max_chunks * 4;
  L.c_pairs = align256(off);
  off = L.c_pairs + L.max_chunks * kChunkCols * 4;
  L.end = align256(off);
  return L;
}

Table table_at(uint8_t* base, const UnitsLayout& L) {
  Table t;
  t.hdr = reinterpret_cast<int32_t*>(base + L.hdr);
  t.unit_expert = reinterpret_cast<int32_t*>(base + L.unit_expert);
  t.unit_rows = reinterpret_cast<int32_t*>(base + L.unit_rows);
  t.g_expert = reinterpret_cast<int32_t*>(base + L.g_expert);
  t.g_unit0 = reinterpret_cast<int32_t*>(base + L.g_unit0);
  t.g_nunits = reinterpret_cast<int32_t*>(base + L.g_nunits);
  t.g_tile0 = reinterpret_cast<int32_t*>(base + L.g_tile0);
  t.c_expert = reinterpret_cast<int32_t*>(base + L.c_expert);
  t.c_cols = reinterpret_cast<int32_t*>(base + L.c_cols);
  t.c_pairs = reinterpret_cast<int32_t*>(base + L.c_pairs);
  return t;
}

// ------------------------------------------------------------------ group
constexpr int kGroupParts = 8;  // workgroups that build the unit table together

// Inclusive scan over a wave (64 lanes).
__device__ __forceinline__ uint32_t wave_scan_u32(uint32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t o = __shfl_up(v, d);
    if (lane >= d) v += o;
  }
  return v;
}

// LDS words of the unit-table build: per-expert token bitmasks (word-major, [W][E]),
// route counts, first unit and first chunk per expert, and the column count of every
// chunk.
size_t group_lds_words(int B, int K, int E) {
  const int64_t U = static_cast<int64_t>(B) * K;
  return static_cast<size_t>(E) * ((B + 31) / 32) + 3 * static_cast<size_t>(E) +
         static_cast<size_t>(max_chunks_for(U, U < E ? U : E));
}

// The unit table (experts page, ExpertsKernel.group / ExpertsGroupKernel): per-expert
// token bitmasks, ceil(n/8) units per expert numbered in expert order, unit rows holding
// pair indices in token order (-1 padded), the list of distinct experts with their first
// unit and 16-column tile offset, and the 32-route chunks.  Built by `parts` workgroups
// of kGroupThreads: every one counts all routes and scans all experts (E <= 1024: thread
// e holds expert e), then writes the per-expert entries of the experts [lo, hi) and the
// unit-row and chunk entries of the routes [r_lo, r_hi), so that each issues 1/parts of
// the table's scattered stores.
__device__ __forceinline__ void group_body(const int32_t* __restrict__ ids, int B, int K, int E, int W, Table tbl,
                                           int part, int parts) {
  extern __shared__ uint32_t lds[];
  constexpr int kPer = 8;  // routes per thread held in registers (all of them for U <= 8192)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int U = B * K;
  const int lo = static_cast<int>(static_cast<int64_t>(part) * E / parts);
  const int hi = static_cast<int>(static_cast<int64_t>(part + 1) * E / parts);
  const int r_lo = static_cast<int>(static_cast<int64_t>(part) * U / parts);
  const int r_hi = static_cast<int>(static_cast<int64_t>(part + 1) * U / parts);
  int ev[kPer];  // requested before anything else
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int r = tid + i * kGroupThreads;
    ev[i] = r < U ? ids[r] : -1;
  }
  uint32_t* masks = lds;                                                     // [W][E]
  int* routes = reinterpret_cast<int*>(masks + static_cast<size_t>(E) * W);  // [E] route counts
  int* unit0 = routes + E;                                                   // [E]
  int* chunk0 = unit0 + E;                                                   // [E]
  int* ncols = chunk0 + E;                                                   // [chunks]
  __shared__ uint32_t wsum[3][kGroupThreads / 64];
  __shared__ uint32_t s_tot[3];
  __shared__ int flags, s_c_lo, s_c_hi;
  for (int i = tid; i < E * W; i += kGroupThreads) masks[i] = 0;
  for (int i = tid; i < E; i += kGroupThreads) routes[i] = 0;
  if (tid == 0) flags = 0;
  __syncthreads();
  // the token of route r, r / K, as a multiply-high: exact, since the error of kinv is
  // below 2^-32 K and r < 2^16
  const uint64_t kinv = (uint64_t{1} << 32) / static_cast<uint64_t>(K) + 1u;
  auto token = [&](int r) { return static_cast<int>((static_cast<uint64_t>(r) * kinv) >> 32); };
  int bad = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int r = tid + i * kGroupThreads;
    if (r < U) {
      const int e = ev[i];
      if (e < 0 || e >= E) {
        bad = 1;
      } else {
        const int t = token(r);
        atomicOr(&masks[(t >> 5) * E + e], 1u << (t & 31));
        atomicAdd(&routes[e], 1);
      }
    }
  }
  for (int r = tid + kPer * kGroupThreads; r < U; r += kGroupThreads) {
    const int e = ids[r];
    if (e < 0 || e >= E) {
      bad = 1;
      continue;
    }
    const int t = token(r);
    atomicOr(&masks[(t >> 5) * E + e], 1u << (t & 31));
    atomicAdd(&routes[e], 1);
  }
  if (bad) atomicOr(&flags, 1);
  __syncthreads();
  // thread e: expert e's route count (token bits; a repeated id sets one bit twice), its
  // units, chunks and 32-column tiles, scanned over the expert waves in two words of two
  // 16-bit fields (units <= E + U/8 and chunks <= E + U/32 stay below 2^16, so no field
  // carries into the next)
  const int ew = (E + 63) >> 6;
  int cnt = 0, units = 0, chunks = 0, grp = 0, tiles = 0;
  uint32_t s0 = 0, s1 = 0, s2 = 0;
  if (wave < ew) {
    if (tid < E) {
      int c0 = 0, c1 = 0, c2 = 0, c3 = 0, w = 0;
      for (; w + 4 <= W; w += 4) {
        c0 += __popc(masks[w * E + tid]);
        c1 += __popc(masks[(w + 1) * E + tid]);
        c2 += __popc(masks[(w + 2) * E + tid]);
        c3 += __popc(masks[(w + 3) * E + tid]);
      }
      for (; w < W; ++w) c0 += __popc(masks[w * E + tid]);
      cnt = c0 + c1 + c2 + c3;
      if (cnt != routes[tid]) atomicOr(&flags, 2);  // an id repeated within a token
    }
    units = (cnt + 7) >> 3;
    chunks = (cnt + kChunkCols - 1) / kChunkCols;
    grp = cnt > 0 ? 1 : 0;
    tiles = (units + 1) >> 1;
    s0 = wave_scan_u32(static_cast<uint32_t>(units) | (static_cast<uint32_t>(grp) << 16));
    s1 = wave_scan_u32(static_cast<uint32_t>(tiles) | (static_cast<uint32_t>(chunks) << 16));
    s2 = wave_scan_u32(static_cast<uint32_t>(cnt));
    if (lane == 63) {
      wsum[0][wave] = s0;
      wsum[1][wave] = s1;
      wsum[2][wave] = s2;
    }
  }
  __syncthreads();
  if (wave < ew) {
    for (int w = 0; w < wave; ++w) {
      s0 += wsum[0][w];
      s1 += wsum[1][w];
      s2 += wsum[2][w];
    }
    const int iu = static_cast<int>(s0 & 0xffffu), ig = static_cast<int>(s0 >> 16);
    const int it = static_cast<int>(s1 & 0xffffu), ic = static_cast<int>(s1 >> 16);
    const int u0 = iu - units, gi = ig - grp, t0 = it - tiles, c0 = ic - chunks;
    if (tid < E) {
      unit0[tid] = u0;
      chunk0[tid] = c0;
    }
    if (tid == E - 1) {
      s_tot[0] = s0;
      s_tot[1] = s1;
      s_tot[2] = s2;
    }
    if (tid == lo) s_c_lo = c0;
    if (tid == hi - 1) s_c_hi = ic;
    if (tid >= lo && tid < hi) {
      for (int q = 0; q < chunks; ++q) {
        const int nc = cnt - q * kChunkCols < kChunkCols ? cnt - q * kChunkCols : kChunkCols;
        ncols[c0 + q] = nc;
        tbl.c_expert[c0 + q] = tid;
        tbl.c_cols[c0 + q] = (static_cast<int>(s2) - cnt + q * kChunkCols) | (nc << 20);
      }
      if (cnt > 0) {
        tbl.g_expert[gi] = tid;
        tbl.g_unit0[gi] = u0;
        tbl.g_nunits[gi] = units;
        tbl.g_tile0[gi] = t0;
        for (int u = 0; u < units; ++u) tbl.unit_expert[u0 + u] = tid;
        for (int sl = cnt & 7; sl != 0 && sl < 8; ++sl) tbl.unit_rows[(u0 + units - 1) * 8 + sl] = -1;
      }
    }
  }
  __syncthreads();
  if (part == 0 && tid == 0) {
    tbl.hdr[0] = static_cast<int>(s_tot[0] & 0xffffu);
    tbl.hdr[1] = static_cast<int>(s_tot[0] >> 16);
    tbl.hdr[2] = static_cast<int>(s_tot[1] & 0xffffu);
    tbl.hdr[3] = flags;
    tbl.hdr[4] = static_cast<int>(s_tot[1] >> 16);
    tbl.hdr[5] = static_cast<int>(s_tot[2]);
  }
  // unit-row and chunk entries of the routes [r_lo, r_hi): rank = the route's position
  // among its expert's routes in token order
  auto place = [&](int r, int e) {
    if (e < 0 || e >= E) return;
    const int t = token(r), tw = t >> 5;
    int rank = __popc(masks[tw * E + e] & ((1u << (t & 31)) - 1u));
    for (int w = 0; w < tw; ++w) rank += __popc(masks[w * E + e]);
    tbl.unit_rows[(unit0[e] + (rank >> 3)) * 8 + (rank & 7)] = r;
    tbl.c_pairs[(chunk0[e] + rank / kChunkCols) * kChunkCols + rank % kChunkCols] = r;
  };
  if (U <= kPer * kGroupThreads) {  // every route is in a thread's registers
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int r = tid + i * kGroupThreads;
      if (r >= r_lo && r < r_hi) place(r, ev[i]);
    }
  } else {
    for (int r = r_lo + tid; r < r_hi; r += kGroupThreads) place(r, ids[r]);
  }
  // chunk pads of the experts [lo, hi): their chunks are contiguous
  if (lo < hi) {
    const int c_lo = s_c_lo, c_hi = s_c_hi;
    for (int idx = c_lo * kChunkCols + tid; idx < c_hi * kChunkCols; idx += kGroupThreads)
      if ((idx & (kChunkCols - 1)) >= ncols[idx / kChunkCols]) tbl.c_pairs[idx] = -1;
  }
}

__global__ __launch_bounds__(kGroupThreads) void group_kernel(const int32_t* __restrict__ ids, int B,
                                                              int K, int E, int W, Table tbl) {
  group_body(ids, B, K, E, W, tbl, blockIdx.x, gridDim.x);
}

// The plan and the unit table of a batch in one launch (moe_plan_group): the first
// kGroupParts workgroups build the unit table, the others quantize x, kGroupThreads / 4
// 32-element blocks each.
__global__ __launch_bounds__(kGroupThreads) void plan_group_kernel(const uint8_t* __restrict__ x, int64_t nblocks,
                                                                   uint8_t* __restrict__ codes,
                                                                   uint8_t* __restrict__ scales,
                                                                   const int32_t* __restrict__ ids, int B, int K,
                                                                   int E, int W, Table tbl) {
  if (blockIdx.x < kGroupParts) {
    group_body(ids, B, K, E, W, tbl, blockIdx.x, kGroupParts);
    return;
  }
  // four lanes per block: a block's lanes are in one wave, and all four are in range or none
  const int64_t idx4 = static_cast<int64_t>(blockIdx.x - kGroupParts) * kGroupThreads + threadIdx.x;
  if (idx4 < 4 * nblocks) plan_quarter(x, idx4, codes, scales);
}

// ------------------------------------------------------------------ packing
// Packed FC1 weights: per (expert e, hidden block j of 32, K step s of 128) four 16-row
// tiles -- gate rows 32j..32j+15, 32j+16..+31, then the same up rows (I + ...) -- each
// one contiguous KB: lane l's 16 bytes are row (l % 16), K-block 4s + l/16, i.e. the
// FP4 A operand of v_mfma_scale_f32_16x16x128_f8f6f4 for that lane.
__device__ __forceinline__ int w13_row(int I, int j, int rt, int l) {
  return (rt < 2 ? 32 * j + 16 * rt : I + 32 * j + 16 * (rt - 2)) + (l & 15);
}

__global__ void pack_w13_codes(const uint4* __restrict__ src, uint4* __restrict__ dst, int E, int D, int I) {
  const int HB = I / 32, NS = D / 128;
  const int64_t total = static_cast<int64_t>(E) * HB * NS * 256;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= total) return;
  const int l = idx & 63, rt = (idx >> 6) & 3;
  const int64_t rest = idx >> 8;
  const int s = rest % NS;
  const int j = (rest / NS) % HB;
  const int e = rest / (static_cast<int64_t>(NS) * HB);
  const int r = w13_row(I, j, rt, l);
  const int kb = 4 * s + (l >> 4);
  dst[idx] = src[(static_cast<int64_t>(e) * 2 * I + r) * (D / 32) + kb];
}

// Packed FC1 scales: per (e, j, K step s, lane l) one word whose byte rt is the E8M0 of
// (row w13_row(rt, l), K-block 4s + l/16): the A scales of one step's four row tiles.
__global__ void pack_w13_scales(const uint8_t* __restrict__ src, uint32_t* __restrict__ dst, int E, int D,
                                int I) {
  const int HB = I / 32, NS = D / 128;
  const int64_t total = static_cast<int64_t>(E) * HB * NS * 64;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= total) return;
  const int l = idx & 63;
  const int64_t rest = idx >> 6;
  const int s = rest % NS;
  const int j = (rest / NS) % HB;
  const int e = rest / (static_cast<int64_t>(NS) * HB);
  uint32_t word = 0;
  for (int rt = 0; rt < 4; ++rt) {
    const int r = w13_row(I, j, rt, l);
    word |= static_cast<uint32_t>(src[(static_cast<int64_t>(e) * 2 * I + r) * (D / 32) + 4 * s + (l >> 4)]) << (8 * rt);
  }
  dst[idx] = word;
}

// Packed FC2 weights: per (expert, 16-row tile of outputs, K step of 128 over I) one KB;
// K beyond I (I not a multiple of 128) is zero-padded.
__global__ void pack_w2_codes(const uint4* __restrict__ src, uint4* __restrict__ dst, int E, int D, int I) {
  const int NS = (I + 127) / 128, HB = I / 32;
  const int64_t total = static_cast<int64_t>(E) * (D / 16) * NS * 64;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= total) return;
  const int l = idx & 63;
  const int64_t rest = idx >> 6;
  const int s = rest % NS;
  const int64_t tile = rest / NS;                  // e * (D/16) + rt2
  const int e = tile / (D / 16), rt2 = tile % (D / 16);
  const int d = 16 * rt2 + (l & 15);
  const int kb = 4 * s + (l >> 4);
  dst[idx] = kb < HB ? src[(static_cast<int64_t>(e) * D + d) * HB + kb] : make_uint4(0, 0, 0, 0);
}

__global__ void pack_w2_scales(const uint8_t* __restrict__ src, uint32_t* __restrict__ dst, int E, int D,
                               int I) {
  const int NS = (I + 127) / 128, NQ = (NS + 3) / 4, HB = I / 32;
  const int64_t total = static_cast<int64_t>(E) * (D / 16) * NQ * 64;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= total) return;
  const int l = idx & 63;
  const int64_t rest = idx >> 6;
  const int q = rest % NQ;
  const int64_t tile = rest / NQ;
  const int e = tile / (D / 16), rt2 = tile % (D / 16);
  const int d = 16 * rt2 + (l & 15);
  uint32_t word = 0;
  for (int i = 0; i < 4; ++i) {
    const int kb = 4 * (4 * q + i) + (l >> 4);
    const uint32_t b = kb < HB ? src[(static_cast<int64_t>(e) * D + d) * HB + kb] : 127u;
    word |= b << (8 * i);
  }
  dst[idx] = word;
}

// ------------------------------------------------------------------ experts
// Workspace of the experts kernel (caller-owned, zeroed once): per-workgroup call
// counters kept in lockstep, per-hidden-block arrival counters (self-resetting) and
// ready flags (tagged with the call number, so they never need a reset), the hidden
// images that FC2 reads, and the split-block FP32 partial sums.
constexpr int kMaxGrid = 2048;     // workgroups of the persistent grid (call counters)
constexpr int kMaxGroups = 1024;   // distinct experts per call (E <= 1024)

struct WsLayout {
  size_t calls, status, arrive, flags, hcodes, hscales, partials;
  size_t qcalls, qclaims, qhq;  // decode form with whole-K FC1 blocks
  size_t gcalls, gflags, ghid;  // grouped form with whole-K FC1 blocks
  size_t gplan, gpflags;        // the grouped form in one launch: its plan, its plan flags
  size_t end;
  int64_t max_tiles, max_blocks;
  int64_t dec_slots;  // decode-form partial-sum slots (512 tagged pairs each)
  int nt_cap;
};

// Decode form (B <= kDecodeMax): at most 8 token columns per expert.
constexpr int kDecodeMax = 8;

// 16-column tiles of all expert groups of a batch: sum_g ceil(n_g / 16) with
// sum_g n_g = U over at most min(E, U) groups.
int64_t max_tiles_for(int64_t U, int E) {
  const int64_t G = U < E ? U : E;
  return (U + 15 * G + 15) / 16;
}


WsLayout ws_layout(int E, int D, int I, int K, int B_max) {
  WsLayout L{};
  const int64_t U = static_cast<int64_t>(B_max) * K;
  const int HB = I / 32;
  const int64_t IP = (I + 127) / 128 * 128;
  L.max_tiles = max_tiles_for(U, E);
  L.max_blocks = L.max_tiles * HB;
  L.nt_cap = 1;  // one 16-column tile per weight pass
  size_t off = 0;
  L.calls = off;
  off = align256(off + kMaxGrid * 4);
  L.status = off;  // the decode form's status word (when the caller passes none)
  off = align256(off + 4);
  L.arrive = off;
  off = align256(off + L.max_blocks * 4);
  L.flags = off;
  off = align256(off + L.max_blocks * 4);
  L.hcodes = off;
  off = align256(off + L.max_tiles * 16 * IP);
  L.hscales = off;
  off = align256(off + L.max_tiles * 16 * (IP / 32));
  // FC1 partial sums: the grouped form's per-workgroup slots, or the decode form's
  // tagged slots -- at most (blocks of a call) + 4 * grid of them
  const int64_t Bd = B_max < kDecodeMax ? B_max : kDecodeMax;
  const int64_t Gd = Bd * K < E ? Bd * K : E;
  L.dec_slots = Gd * HB + 4 * static_cast<int64_t>(kMaxGrid) + 4;
  const size_t grouped = static_cast<size_t>(kMaxGrid) * 4 * L.nt_cap * 4096;
  const size_t dec = static_cast<size_t>(L.dec_slots) * 4096;
  L.partials = off;
  off = align256(off + (grouped > dec ? grouped : dec));
  // decode form with whole-K FC1 blocks: its own call counters and the hidden as
  // (data, call) pairs (at most 128 distinct experts x 8 token columns x (IP/4 + 16))
  L.qcalls = off;
  off = align256(off + kMaxGrid * 4);
  L.qclaims = off;  // FC2 claim counters, one per workgroup (call-tagged: never cleared)
  off = align256(off + kMaxGrid * 8);
  L.qhq = off;
  off = align256(off + static_cast<size_t>(128) * 8 * (IP / 4 + 16) * 8);
  // grouped form with whole-K FC1 blocks: its call counters, a call-tagged flag per
  // (chunk, hidden block) and the published hidden, [chunk][32 columns][IP + 16] (plus 1
  // KB that the loader's 1 KB DMA pieces may read past the last chunk)
  const int64_t chunks = max_chunks_for(U, U < E ? U : E);
  L.gcalls = off;
  off = align256(off + kMaxGrid * 4);
  L.gflags = off;
  off = align256(off + static_cast<size_t>(chunks) * HB * 4);
  L.ghid = off;
  off = align256(off + static_cast<size_t>(chunks) * kChunkCols * (IP + 16) + 1024);
  // the grouped form in one launch (moe_decode_run, B > 8): the plan it makes (x codes,
  // then scales) and a call-tagged flag per workgroup for its share
  L.gplan = off;
  off = align256(off + static_cast<size_t>(B_max) * D / 32 * 33);
  L.gpflags = off;
  off = align256(off + kMaxGrid * 4);
  L.end = off;
  return L;
}

struct ExpArgs {
  const uint8_t* w13p;
  const uint8_t* s13p;
  const uint8_t* w2p;
  const uint8_t* s2p;
  const uint8_t* xcodes;
  const uint8_t* xscales;
  Table tbl;
  uint32_t* calls;
  uint32_t* arrive;
  uint32_t* flags;
  uint8_t* hcodes;
  uint8_t* hscales;
  float* partials;
  uint16_t* out;
  uint8_t* dump_codes;
  uint8_t* dump_scales;
  int D, I, HB, NS1, IP, K, floor_rule;
  int NSP;  // FC1 items per hidden block: pairs of 128-wide K steps (NS1 / 2)
  uint32_t plan_bytes;  // bytes of the plan (x codes, then x scales)
  int U2;   // FC2 items per chunk: groups of T2 16-row output tiles (D / 16 / T2)
  int g_cap, u_cap;  // LDS capacity of the group list and the unit rows
  int32_t* err;      // status word: bit 0 id out of range, bit 1 id repeated in a token,
                     // bit 2 a wait gave up (never expected)
  // decode form (B <= 8): routing and the MXFP8 plan of x happen in the kernel
  const uint16_t* x;     // BF16 [B, D]
  const int32_t* ids;    // [B, K]
  uint8_t* plan_dump;    // optional: the plan of x in the moe_plan layout (workgroup 0)
  uint64_t* dpart;       // call-tagged FC1 partial sums: (float bits, call + 1) pairs
  int B, E;
  int qmin;  // decode form: least FC1 items per workgroup slice (0: grouped form)
};

// ------------------------------------------------------------ LDS access
// The weight stream reaches LDS by DMA (global_load_lds); the compiler's wait-count
// pass cannot tell those writes from other LDS data and would drain the whole stream
// before every LDS read.  Every LDS access after the first DMA therefore goes through
// these asm helpers, which wait for their own completion (lgkmcnt) only; the stream's
// completion is awaited explicitly (vmcnt) where a slot is consumed.
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ uint4 lds_ld16(uint32_t addr) {
  uint4 v;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return v;
}
__device__ __forceinline__ uint32_t lds_ld4(uint32_t addr) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return v;
}
__device__ __forceinline__ uint32_t lds_ld2(uint32_t addr) {
  uint32_t v;
  asm volatile("ds_read_u16 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return v;
}
__device__ __forceinline__ void lds_st16(uint32_t addr, uint4 v) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  const v4u x = {v.x, v.y, v.z, v.w};
  asm volatile("ds_write_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : : "v"(addr), "v"(x) : "memory");
}
// Four 16-byte reads at addr + k * stride (one wait for all four).
template <int OFF, int STRIDE>
__device__ __forceinline__ void lds_ld16x4(uint32_t addr, uint4& v0, uint4& v1, uint4& v2, uint4& v3) {
  asm volatile(
      "ds_read_b128 %0, %4 offset:%5\n\t"
      "ds_read_b128 %1, %4 offset:%6\n\t"
      "ds_read_b128 %2, %4 offset:%7\n\t"
      "ds_read_b128 %3, %4 offset:%8\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3)
      : "v"(addr), "n"(OFF), "n"(OFF + STRIDE), "n"(OFF + 2 * STRIDE), "n"(OFF + 3 * STRIDE)
      : "memory");
}
// Four 4-byte reads at addr + k * stride.
template <int OFF, int STRIDE>
__device__ __forceinline__ void lds_ld4x4(uint32_t addr, uint32_t& v0, uint32_t& v1, uint32_t& v2, uint32_t& v3) {
  asm volatile(
      "ds_read_b32 %0, %4 offset:%5\n\t"
      "ds_read_b32 %1, %4 offset:%6\n\t"
      "ds_read_b32 %2, %4 offset:%7\n\t"
      "ds_read_b32 %3, %4 offset:%8\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3)
      : "v"(addr), "n"(OFF), "n"(OFF + STRIDE), "n"(OFF + 2 * STRIDE), "n"(OFF + 3 * STRIDE)
      : "memory");
}
// Two 16-byte reads and one 4-byte read (a token tile's B operand and its scale word).
template <int OFF_LO, int OFF_HI, int OFF_S>
__device__ __forceinline__ void lds_ld_b(uint32_t addr16, uint32_t addr4, uint4& lo, uint4& hi, uint32_t& sw) {
  asm volatile(
      "ds_read_b128 %0, %3 offset:%5\n\t"
      "ds_read_b128 %1, %3 offset:%6\n\t"
      "ds_read_b32 %2, %4 offset:%7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(lo), "=&v"(hi), "=&v"(sw)
      : "v"(addr16), "v"(addr4), "n"(OFF_LO), "n"(OFF_HI), "n"(OFF_S)
      : "memory");
}
// Uniform (same address in every lane) LDS word, moved to a scalar register.
__device__ __forceinline__ int lds_uni(uint32_t addr) {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(lds_ld4(addr)));
}

template <int VMCNT>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(VMCNT) : "memory");
}

__device__ __forceinline__ void dma16(const void* g, uint32_t lds_off) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __builtin_amdgcn_global_load_lds(g, (lds_void*)(smem + lds_off), 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds_off) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __builtin_amdgcn_global_load_lds(g, (lds_void*)(smem + lds_off), 4, 0, 0);
}
// The same with the non-temporal hint (cache policy NT): for data read exactly once
// (the weight stream), so that its lines are the first the L2 evicts and do not push
// out data that other workgroups read again.
constexpr int kNT = 2;
__device__ __forceinline__ void dma16_nt(const void* g, uint32_t lds_off) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __builtin_amdgcn_global_load_lds(g, (lds_void*)(smem + lds_off), 16, 0, kNT);
}
__device__ __forceinline__ void dma4_nt(const void* g, uint32_t lds_off) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __builtin_amdgcn_global_load_lds(g, (lds_void*)(smem + lds_off), 4, 0, kNT);
}
// DMA through a buffer resource: lanes whose offset lies outside the buffer write zeros
// and read no memory (a padded column, or a pad that only keeps the DMA count fixed).
constexpr uint32_t kOutside = 0x80000000u;
__device__ __forceinline__ void bdma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds_off) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(smem + lds_off), 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void bdma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds_off) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(smem + lds_off), 4, voff, 0, 0, 0);
}
// DMA through a buffer resource with the lane's offset `voff` (a loop-invariant register)
// and a scalar offset `soff`: a stream of such loads needs no vector address arithmetic
// between them (a vector register that a load has not yet read holds up the instruction
// that would overwrite it).  A lane whose voff lies outside the buffer writes zeros.
template <int AUX = 0>
__device__ __forceinline__ void sdma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t lds_off) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(smem + lds_off), 16, voff, soff, 0, AUX);
}
template <int AUX = 0>
__device__ __forceinline__ void sdma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t lds_off) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(smem + lds_off), 4, voff, soff, 0, AUX);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}

// The wave's index in its workgroup, as a scalar (uniform) value: derived from
// threadIdx.x the compiler would keep it, and everything computed from it, per lane.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6)); }
__device__ __forceinline__ uint32_t lds_base() {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  return static_cast<uint32_t>(reinterpret_cast<size_t>((lds_void*)smem));
}
__device__ __forceinline__ void lds_settle_all() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void lds_st4(uint32_t addr, uint32_t v) {
  asm volatile("ds_write_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : : "v"(addr), "v"(v) : "memory");
}

// Waits (bounded, tens of milliseconds) until the LDS word at addr reaches `want`
// (>= or ==).  The waves of a workgroup hand work to each other through such words; a
// wait that runs out sets bit 2 of the unit-table flags and goes on.
template <bool EQ>
__device__ __forceinline__ void lds_wait(uint32_t addr, int want, int32_t* err) {
  #pragma unroll 1
  for (uint32_t spins = 0;; ++spins) {
    const int v = lds_uni(addr);
    if (EQ ? v == want : v >= want) return;
    if (spins == kSpinLimit) {
      if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_or(err, 4, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// ------------------------------------------------------------ LDS layout
// [groups: g_cap records {expert, unit0, nunits, tile0}]  [chunk0: g_cap + 1 words]
// [unit rows: u_cap x 8 u16 pair indices, 0xffff = padding]  [sync words]  [slice table]  [red: 2 x 4 streaming waves x NT x 4 KB, later reused as the 2 hidden
// buffers]  [meta: 4 waves x R x 16 B]  [ring: 4 waves x R x slot]
// FC2 output tiles per item, so that an FC2 item carries about as many weight bytes as
// an FC1 item.
template <int NS2>
struct Fc2Tiles {
  static constexpr int T2 = NS2 == 1 ? 8 : (NS2 == 2 ? 4 : 2);
};

// Ring geometry.  Grouped form: an FC1 item carries its x operand (13 KB slot).  Decode
// form (DEC): x sits in LDS for the whole call, so a slot holds only weights: the FC1
// item (8.5 KB) or the FC2 item (A codes, then its scale words from byte 8192).  Items
// that issue fewer than L DMA instructions pad with zero-filling word loads from
// outside a buffer into the slot's pad area, which nothing reads.
template <int NT, int R_, int NS2, bool DEC>
struct Geo {
  static constexpr int R = R_;                               // items in flight per wave
  static constexpr int T2 = Fc2Tiles<NS2>::T2;
  static constexpr int FC2_END = 8192 + T2 * 256;            // end of an FC2 item's scale words
  static constexpr int SLOT = DEC ? (FC2_END > 8704 ? FC2_END : 8704) + 256 : 13312;
  static constexpr int PAD = DEC ? SLOT - 256 : 12800;
  static constexpr int L = DEC ? (T2 * NS2 + T2 > 10 ? T2 * NS2 + T2 : 10) : 16;  // DMA instructions per item
  static constexpr int VM = (R - 1) * L;                     // vmcnt that completes the oldest of R items
  static constexpr int RED = 2 * kStream * NT * 4096;  // two hand-over slots per wave
};

// Sync words (u32, offsets within the sync area): sub[w] = FC1 blocks wave w has handed
// over; ack = blocks the control wave has taken; prog[w] = the FC2 chunk (index in the
// workgroup's sequence) wave w works on; ready[b] = the chunk held by hidden buffer b;
// x = 1 once the decode form's plan of x is in LDS.
constexpr uint32_t kSyncSub = 0, kSyncAck = 16, kSyncProg = 32, kSyncReady = 48, kSyncX = 56, kSyncBytes = 64;

struct LdsMap {
  uint32_t grec, chunk0, urows, sync, slt, red, hid, hid_bytes, hs, meta, ring;
  uint32_t xq, xs, xstr, xss;  // decode form: x codes [B + 1 rows of xstr], x scales [B + 1 rows of xss]
  uint32_t scr;                // decode form: the hidden builder's staging area (in red)
};

// Decode form: the hidden builder stages up to kRound tagged partial sums per lane.
constexpr int kRound = 16;

// Hidden buffer of one FC2 chunk: NT*16 columns x (IP + 16) code bytes (padded rows),
// then NT*16 columns x IP/32 scale bytes.  The two hidden buffers share the FC1
// hand-over area: the control wave fills them only after it took every FC1 block.
// Decode form: x codes rows are D + 16 bytes apart (the rows of different tokens then
// start in different LDS banks), scale rows D/32 + 4; row B is all zeros and stands in
// for padded columns.  In red, after the two hidden buffers: the hidden builder's
// staging area (kRound x 64 words) and its per-chunk table (96 words).
template <int NT, int R, int NS2, bool DEC>
__host__ __device__ __forceinline__ LdsMap lds_map(uint32_t g_cap, uint32_t u_cap, uint32_t IP, uint32_t B,
                                                   uint32_t D) {
  using G = Geo<NT, R, NS2, DEC>;
  LdsMap t;
  t.grec = 0;
  t.chunk0 = g_cap * 16;
  t.urows = (t.chunk0 + (g_cap + 1) * 4 + 15) & ~15u;
  t.sync = t.urows + u_cap * 16;
  t.slt = t.sync + kSyncBytes;  // the workgroup's four slices, 32 bytes each
  t.red = t.slt + 128;
  t.hs = IP + 16;
  t.hid_bytes = (NT * 16 * t.hs + NT * 16 * (IP / 32) + 15) & ~15u;
  t.hid = t.red;
  t.scr = t.red + 2 * t.hid_bytes;
  const uint32_t need = DEC ? 2 * t.hid_bytes + kRound * 256 + 384 : 2 * t.hid_bytes;
  const uint32_t area = need > static_cast<uint32_t>(G::RED) ? need : static_cast<uint32_t>(G::RED);
  t.meta = t.red + ((area + 15) & ~15u);
  t.xq = t.meta + kStream * R * 16;
  t.xstr = D + 16;
  t.xss = D / 32 + 4;
  t.xs = t.xq + (DEC ? (B + 1) * t.xstr : 0);
  t.ring = (t.xs + (DEC ? (B + 1) * t.xss : 0) + 15) & ~15u;
  return t;
}

template <int NT, int R, int NS2, bool DEC>
inline size_t lds_bytes(int g_cap, int u_cap, int IP, int B, int D) {
  const LdsMap t = lds_map<NT, R, NS2, DEC>(static_cast<uint32_t>(g_cap), static_cast<uint32_t>(u_cap),
                                            static_cast<uint32_t>(IP), static_cast<uint32_t>(B),
                                            static_cast<uint32_t>(D));
  return t.ring + kStream * static_cast<size_t>(R) * Geo<NT, R, NS2, DEC>::SLOT;
}

// Per-workgroup copy of the unit table: the group list, chunk0[g] = first weight-pass
// chunk of group g (chunks of NT column tiles; chunk0[n_groups] = total), and the unit
// rows as 16-bit pair indices.  Plain LDS stores: this runs before the first DMA.
template <int NT>
__device__ __forceinline__ int load_groups(const ExpArgs& a, const LdsMap& m, int n_groups, int n_units) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int4* grec = reinterpret_cast<int4*>(smem + m.grec);
  int* chunk0 = reinterpret_cast<int*>(smem + m.chunk0);
  uint16_t* urows = reinterpret_cast<uint16_t*>(smem + m.urows);
  if (threadIdx.x < kSyncBytes / 4) {
    const int i = threadIdx.x;  // sub, ack = 0; prog, ready = -1
    reinterpret_cast<int*>(smem + m.sync)[i] = (i * 4 >= static_cast<int>(kSyncProg)) ? -1 : 0;
  }
  for (int i = threadIdx.x; i < n_groups; i += kWG)
    grec[i] = make_int4(a.tbl.g_expert[i], a.tbl.g_unit0[i], a.tbl.g_nunits[i], a.tbl.g_tile0[i]);
  // unit rows: int32 pair indices (-1 = padding) -> u16; four units per thread in flight
  const int4* rows = reinterpret_cast<const int4*>(a.tbl.unit_rows);
  for (int base = 0; base < n_units; base += 4 * kWG) {
    int4 r[4][2];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int u = base + q * kWG + static_cast<int>(threadIdx.x);
      if (u < n_units) {
        r[q][0] = rows[2 * u];
        r[q][1] = rows[2 * u + 1];
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int u = base + q * kWG + static_cast<int>(threadIdx.x);
      if (u < n_units) {
        auto pk = [](int lo, int hi) {
          return (static_cast<uint32_t>(lo) & 0xffffu) | (static_cast<uint32_t>(hi) << 16);
        };
        *reinterpret_cast<uint4*>(urows + 8 * u) = make_uint4(pk(r[q][0].x, r[q][0].y), pk(r[q][0].z, r[q][0].w),
                                                              pk(r[q][1].x, r[q][1].y), pk(r[q][1].z, r[q][1].w));
      }
    }
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int carry = 0;
    for (int base = 0; base < n_groups; base += 64) {
      const int g = base + lane;
      const int v = g < n_groups ? (((grec[g].z + 1) >> 1) + NT - 1) / NT : 0;
      int inc = v;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(inc, d);
        if (lane >= d) inc += o;
      }
      if (g < n_groups) chunk0[g] = carry + inc - v;
      carry += __shfl(inc, 63);
    }
    if (lane == 0) chunk0[n_groups] = carry;
  }
  __syncthreads();
  return chunk0[n_groups];
}

// Exclusive scan of v over the kWG threads of a workgroup (wtot: kWG/64 LDS words);
// `total` gets the sum.  Contains a workgroup barrier.
__device__ __forceinline__ int wg_exclusive_scan(int v, int* wtot, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(inc, d);
    if (lane >= d) inc += o;
  }
  if (lane == 63) wtot[wave] = inc;
  __syncthreads();
  int base = 0;
  total = 0;
#pragma unroll
  for (int ww = 0; ww < kWG / 64; ++ww) {
    const int t = wtot[ww];
    if (ww < wave) base += t;
    total += t;
  }
  return base + inc - v;
}

// MXFP8 of one 32-element BF16 block (w: its 16 words): 8 code words; returns the
// E8M0 exponent (experts page, mx_block; the same arithmetic as plan_kernel).
__device__ __forceinline__ int mx_block32(const uint32_t (&w)[16], uint32_t (&c)[8]) {
  float v[32];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    amax = fmaxf(amax, fmaxf(fabsf(v[2 * i]), fabsf(v[2 * i + 1])));
  }
  const int e = mx_exponent(amax, false);
  const float s = exp2_neg(e);
#pragma unroll
  for (int k = 0; k < 8; ++k)
    c[k] = to_e4m3(v[4 * k] * s) | (to_e4m3(v[4 * k + 1] * s) << 8) | (to_e4m3(v[4 * k + 2] * s) << 16) |
           (to_e4m3(v[4 * k + 3] * s) << 24);
  return e;
}

// Four binary32 values to four e4m3 codes (byte i = value i) with gfx950's packed
// conversion.  It rounds to nearest even like to_e4m3; inputs must lie in [-448, 448]
// (callers clamp or know it), where the two agree on every value (checked exhaustively
// on the device, both signs).
__device__ __forceinline__ uint32_t cvt4_e4m3(float v0, float v1, float v2, float v3) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, lo, true));
}

// mx_block32 with the packed conversion: the default exponent rule bounds every scaled
// value by 448, so no clamp is needed.
__device__ __forceinline__ int mx_block32_hw(const uint32_t (&w)[16], uint32_t (&c)[8]) {
  float v[32];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    amax = fmaxf(amax, fmaxf(fabsf(v[2 * i]), fabsf(v[2 * i + 1])));
  }
  const int e = mx_exponent(amax, false);
  const float s = exp2_neg(e);
#pragma unroll
  for (int k = 0; k < 8; ++k) c[k] = cvt4_e4m3(v[4 * k] * s, v[4 * k + 1] * s, v[4 * k + 2] * s, v[4 * k + 3] * s);
  return e;
}

__device__ __forceinline__ void fill_slices(const ExpArgs& a, const LdsMap& m, int n_groups, int n_chunks);

// Plans of x up to this many 32-element blocks are the control wave's alone (dec_plan_x,
// while the streaming waves start); larger ones are quantized by all waves in the
// prologue.
constexpr int kPlanByControl = 256;

// Decode form prologue, all waves, before the first weight DMA.  Every workgroup builds
// in its own LDS the unit table of the batch (B <= 8; experts page, the capacity <= 8
// path: one unit per distinct expert, experts ascending, its tokens in token order --
// the table moe_group writes for such a batch) and its slice table, so the whole step is
// one launch.  A plan of x larger than kPlanByControl blocks is made here too, by all
// waves (the moe_plan arithmetic; its raw rows come in by DMA into the ring, issued
// first so they travel with the ids); a smaller one is dec_plan_x's.  Returns the number
// of distinct experts.
__device__ __forceinline__ int dec_route(const ExpArgs& a, const LdsMap& m, uint32_t ring_bytes) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x;
  const int U = a.B * a.K, E = a.E, D = a.D, nkb = D / 32, nxb = a.B * nkb;
  const bool plan_here = nxb > kPlanByControl;
  // raw rows of x into the ring behind the routing scratch, as many 1 KB pieces as fit
  // per pass (the first pass is issued before anything waits)
  const int pieces = a.B * D * 2 / 1024, per_pass = static_cast<int>(ring_bytes - 4096) / 1024;
  const int w = wave_id(), l = threadIdx.x & 63;
  const uint8_t* xb = reinterpret_cast<const uint8_t*>(a.x);
  auto stage_x = [&](int p0) {
    const int np = pieces - p0 < per_pass ? pieces - p0 : per_pass;
#pragma unroll 1
    for (int i = w; i < np; i += kWG / 64) dma16(xb + (p0 + i) * 1024 + l * 16, m.ring + 4096 + i * 1024);
  };
  if (plan_here) {
    stage_x(0);
  } else if (w == kStream) {
    // small plan: the control wave's (dec_plan_x); its raw rows go out now, ahead of
    // the weight streams in the memory pipeline, into the idle FC1 hand-over area
#pragma unroll 1
    for (int i = 0; i < pieces; ++i) dma16(xb + i * 1024 + l * 16, m.red + i * 1024);
  }
  // scratch in the ring, which no weight DMA has touched yet: per-expert token masks (a byte
  // per expert), expert -> group rank, wave totals
  uint32_t* mk = reinterpret_cast<uint32_t*>(smem + m.ring);          // [ceil(E / 4)]
  uint16_t* rk = reinterpret_cast<uint16_t*>(smem + m.ring + 1024);   // [E]
  int* wtot = reinterpret_cast<int*>(smem + m.ring + 3072);           // [kWG / 64]
  uint16_t* urows = reinterpret_cast<uint16_t*>(smem + m.urows);
  int4* grec = reinterpret_cast<int4*>(smem + m.grec);
  int* chunk0 = reinterpret_cast<int*>(smem + m.chunk0);
  // the ids (U <= 512: at most 2 per thread)
  int id[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int r = tid + q * kWG;
    id[q] = r < U ? a.ids[r] : -1;
  }
  for (int i = tid; i < (E + 3) / 4; i += kWG) mk[i] = 0u;
  for (int i = tid; i < a.u_cap * 8; i += kWG) urows[i] = 0xffffu;
  if (tid < kSyncBytes / 4)  // sub, ack = 0; prog, ready = -1
    reinterpret_cast<int*>(smem + m.sync)[tid] = (tid * 4 >= static_cast<int>(kSyncProg)) ? -1 : 0;
  for (int i = tid; i < D / 16; i += kWG)
    *reinterpret_cast<uint4*>(smem + m.xq + a.B * m.xstr + 16 * i) = make_uint4(0u, 0u, 0u, 0u);
  for (int i = tid; i < static_cast<int>(m.xss) / 4; i += kWG)
    *reinterpret_cast<uint32_t*>(smem + m.xs + a.B * m.xss + 4 * i) = 0u;
  __syncthreads();
  // token masks; an id repeated within a token finds its bit already set
  int flags = 0;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int r = tid + q * kWG;
    if (r >= U) continue;
    const int e = id[q];
    if (e < 0 || e >= E) {
      flags |= 1;
      continue;
    }
    const uint32_t bit = 1u << ((e & 3) * 8 + r / a.K);
    if (atomicOr(&mk[e >> 2], bit) & bit) flags |= 2;
  }
  __syncthreads();
  // group ranks: thread i takes experts 4i .. 4i+3 (E <= 1024 -> 256 threads)
  const uint32_t mw = tid < (E + 3) / 4 ? mk[tid] : 0u;
  int cnt = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) cnt += ((mw >> (8 * b)) & 0xffu) != 0u;
  int n_groups = 0;
  int g = wg_exclusive_scan(cnt, wtot, n_groups);
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    if (((mw >> (8 * b)) & 0xffu) == 0u) continue;
    const int e = 4 * tid + b;
    rk[e] = static_cast<uint16_t>(g);
    grec[g] = make_int4(e, g, 1, g);  // one unit, one column tile per expert
    chunk0[g] = g;
    ++g;
  }
  if (tid == 0) chunk0[n_groups] = n_groups;
  __syncthreads();
  fill_slices(a, m, n_groups, n_groups);  // one chunk per group; read after the barriers below
  // unit rows: pair r of token t at t's rank among the expert's tokens
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int r = tid + q * kWG;
    const int e = id[q];
    if (r >= U || e < 0 || e >= E) continue;
    const int t = r / a.K;
    const uint32_t tm = (mk[e >> 2] >> ((e & 3) * 8)) & 0xffu;
    urows[rk[e] * 8 + __popc(tm & ((1u << t) - 1u))] = static_cast<uint16_t>(r);
  }
  if (flags && blockIdx.x == 0) __hip_atomic_fetch_or(a.err, flags, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (plan_here) {
#pragma unroll 1
    for (int p0 = 0; p0 < pieces; p0 += per_pass) {
      const int np = pieces - p0 < per_pass ? pieces - p0 : per_pass;
      if (p0 > 0) stage_x(p0);
      wait_vm<0>();
      __syncthreads();
#pragma unroll 1
      for (int blk = p0 * 16 + tid; blk < (p0 + np) * 16; blk += kWG) {
        const uint4* src = reinterpret_cast<const uint4*>(smem + m.ring + 4096 + (blk - p0 * 16) * 64);
        uint32_t xw[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint4 v = src[i];
          xw[4 * i] = v.x; xw[4 * i + 1] = v.y; xw[4 * i + 2] = v.z; xw[4 * i + 3] = v.w;
        }
        uint32_t c[8];
        const int e = mx_block32(xw, c);
        const int t = blk / nkb, kb = blk - t * nkb;
        uint4* dst = reinterpret_cast<uint4*>(smem + m.xq + t * m.xstr + 32 * kb);
        dst[0] = make_uint4(c[0], c[1], c[2], c[3]);
        dst[1] = make_uint4(c[4], c[5], c[6], c[7]);
        smem[m.xs + t * m.xss + kb] = static_cast<unsigned char>(e + 127);
        if (a.plan_dump != nullptr && blockIdx.x == 0) {
          uint4* pd = reinterpret_cast<uint4*>(a.plan_dump + static_cast<int64_t>(blk) * 32);
          pd[0] = make_uint4(c[0], c[1], c[2], c[3]);
          pd[1] = make_uint4(c[4], c[5], c[6], c[7]);
          a.plan_dump[static_cast<int64_t>(nxb) * 32 + blk] = static_cast<uint8_t>(e + 127);
        }
      }
      __syncthreads();
    }
    if (tid == 0) reinterpret_cast<uint32_t*>(smem + m.sync)[kSyncX / 4] = 1u;  // x plan ready
  }
  __syncthreads();  // the unit rows (and the plan) are in place; the ring's scratch is free
  return n_groups;
}


// Decode form, the control wave: the MXFP8 plan of x (the moe_plan arithmetic; at most
// kPlanByControl blocks, i.e. 16 KB of raw rows) into LDS, and the optional plan dump
// (workgroup 0).  dec_route already had the BF16 rows DMA'd into the FC1 hand-over area
// (idle until the first FC1 block is handed over, which needs this plan first); one
// lane per 32-element block.  The streaming waves meanwhile start their weight streams;
// the kSyncX word tells them the plan is there.
__device__ __forceinline__ void dec_plan_x(const ExpArgs& a, const LdsMap& m, uint32_t sy) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int l = threadIdx.x & 63;
  const int D = a.D, nkb = D / 32, nxb = a.B * nkb;
  static_assert(kPlanByControl * 64 <= 32 * 1024, "the raw rows fit the hand-over area");
  wait_vm<0>();
  {
    const int p0 = 0, np = a.B * D * 2 / 1024;
#pragma unroll 1
    for (int blk = p0 * 16 + l; blk < (p0 + np) * 16; blk += 64) {
      const uint4* src = reinterpret_cast<const uint4*>(smem + m.red + (blk - p0 * 16) * 64);
      uint32_t xw[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 v = src[i];
        xw[4 * i] = v.x; xw[4 * i + 1] = v.y; xw[4 * i + 2] = v.z; xw[4 * i + 3] = v.w;
      }
      uint32_t c[8];
      const int e = mx_block32(xw, c);
      const int t = blk / nkb, kb = blk - t * nkb;
      uint4* dst = reinterpret_cast<uint4*>(smem + m.xq + t * m.xstr + 32 * kb);
      dst[0] = make_uint4(c[0], c[1], c[2], c[3]);
      dst[1] = make_uint4(c[4], c[5], c[6], c[7]);
      smem[m.xs + t * m.xss + kb] = static_cast<unsigned char>(e + 127);
      if (a.plan_dump != nullptr && blockIdx.x == 0) {
        uint4* pd = reinterpret_cast<uint4*>(a.plan_dump + static_cast<int64_t>(blk) * 32);
        pd[0] = make_uint4(c[0], c[1], c[2], c[3]);
        pd[1] = make_uint4(c[4], c[5], c[6], c[7]);
        a.plan_dump[static_cast<int64_t>(nxb) * 32 + blk] = static_cast<uint8_t>(e + 127);
      }
    }
  }
  lds_settle_all();
  if (l == 0) lds_st4(sy + kSyncX, 1u);
}

struct GroupInfo {
  int g, c0, c1, cc, e, unit0, nunits, tile0, ntiles;  // c0, c1: the group's chunks [c0, c1)
};

// Fields of group g (uniform LDS words); cc is left to the caller.
__device__ __forceinline__ GroupInfo group_at(const LdsMap& m, uint32_t lb, int g) {
  GroupInfo gi;
  gi.g = g;
  uint4 r;
  uint32_t c0, c1;
  asm volatile(
      "ds_read_b128 %0, %3\n\t"
      "ds_read_b32 %1, %4\n\t"
      "ds_read_b32 %2, %4 offset:4\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r), "=&v"(c0), "=&v"(c1)
      : "v"(lb + m.grec + 16 * g), "v"(lb + m.chunk0 + 4 * g)
      : "memory");
  gi.c0 = __builtin_amdgcn_readfirstlane(static_cast<int>(c0));
  gi.c1 = __builtin_amdgcn_readfirstlane(static_cast<int>(c1));
  gi.e = __builtin_amdgcn_readfirstlane(static_cast<int>(r.x));
  gi.unit0 = __builtin_amdgcn_readfirstlane(static_cast<int>(r.y));
  gi.nunits = __builtin_amdgcn_readfirstlane(static_cast<int>(r.z));
  gi.tile0 = __builtin_amdgcn_readfirstlane(static_cast<int>(r.w));
  gi.ntiles = (gi.nunits + 1) >> 1;
  gi.cc = 0;
  return gi;
}

// The group of weight-pass chunk `chunk` (largest g with chunk0[g] <= chunk).
__device__ __forceinline__ GroupInfo group_of(const LdsMap& m, uint32_t lb, int n_groups, int chunk) {
  int lo = 0, hi = n_groups - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (lds_uni(lb + m.chunk0 + 4 * mid) <= chunk) lo = mid; else hi = mid - 1;
  }
  GroupInfo gi = group_at(m, lb, lo);
  gi.cc = chunk - gi.c0;
  return gi;
}

// Pair index (t*topk + s) of column `col` of a group, or -1 (padding).
__device__ __forceinline__ int column_pair(const LdsMap& m, uint32_t lb, const GroupInfo& gi, int col) {
  const int u = col >> 3;
  if (u >= gi.nunits) return -1;
  const uint32_t v = lds_ld2(lb + m.urows + ((gi.unit0 + u) * 8 + (col & 7)) * 2);
  return v == 0xffffu ? -1 : static_cast<int>(v);
}

// Gated activation and MXFP8 requantization of one 16-column tile of hidden block j
// (experts page, ExpertsKernel.store_hidden: SwiGLU here, FP32 hidden straight from
// the accumulators, one E8M0 exponent per 32 hidden values of a route).
// tot[0], tot[1]: gate rows 0-15 / 16-31 of the block; tot[2], tot[3]: the matching
// up rows.  Lane l holds column l%16, block rows 4*(l/16)+r (+16 for tot[1], tot[3]).
// Called by one whole wave.
__device__ __forceinline__ void hidden_epilogue(const ExpArgs& a, const v4f (&tot)[4], int j, int gtile, int pair) {
  const int l = threadIdx.x & 63;
  float h[2][4];
  float amax = 0.0f;
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float gv = tot[half][r], uv = tot[2 + half][r];
      h[half][r] = gv / (1.0f + expf(-gv)) * uv;
      amax = fmaxf(amax, fabsf(h[half][r]));
    }
  amax = fmaxf(amax, __shfl_xor(amax, 16));
  amax = fmaxf(amax, __shfl_xor(amax, 32));
  const int e = mx_exponent(amax, a.floor_rule != 0);
  const float s = exp2_neg(e);
  uint32_t word[2];
#pragma unroll
  for (int half = 0; half < 2; ++half)
    word[half] = to_e4m3(h[half][0] * s) | (to_e4m3(h[half][1] * s) << 8) |
                 (to_e4m3(h[half][2] * s) << 16) | (to_e4m3(h[half][3] * s) << 24);
  const int gcol = gtile * 16 + (l & 15);
  if (pair >= 0) {  // padded columns: nothing reads their hidden
    uint8_t* hc = a.hcodes + static_cast<int64_t>(gcol) * a.IP + 32 * j + 4 * (l >> 4);
    st_dev_u32(hc, word[0]);
    st_dev_u32(hc + 16, word[1]);
    if (l < 16) st_dev_u8(a.hscales + static_cast<int64_t>(gcol) * (a.IP / 32) + j, static_cast<uint8_t>(e + 127));
  }
  if (a.dump_codes != nullptr && pair >= 0) {
    uint8_t* dc = a.dump_codes + static_cast<int64_t>(pair) * a.I + 32 * j + 4 * (l >> 4);
    *reinterpret_cast<uint32_t*>(dc) = word[0];
    *reinterpret_cast<uint32_t*>(dc + 16) = word[1];
    if (l < 16) a.dump_scales[static_cast<int64_t>(pair) * (a.I / 32) + j] = static_cast<uint8_t>(e + 127);
  }
}

// ------------------------------------------------------------ work partition
// The chunks (groups x weight passes) are split in two halves A and B.  Each workgroup
// walks four contiguous slices, in this order: FC1 steps of A, FC1 steps of B, FC2
// units of A, FC2 units of B (experts page, ExpertsKernel.partition: FC1(A), FC1(B),
// FC2(A), FC2(B)), so that a hidden block is needed only well after the slices that
// produce it ran, and the FC1->FC2 dependency costs no waiting except at the very end.
// An FC1 item is 64 weight rows (gate rows 32j..32j+31 and the matching up rows) x 256
// K (two 128-wide steps) of hidden block j of a chunk; an FC2 item is T2 tiles of 16
// output rows x I of a chunk.
// Global FC1 block numbers run over half A, then half B (chunk * HB + j).

// floor(n / d) for 0 <= n < 2^52, d >= 1: the rounded double quotient is within one.
__device__ __forceinline__ int div_floor(int64_t n, int d) {
  int64_t q = static_cast<int64_t>(static_cast<double>(n) / static_cast<double>(d));
  const int64_t r = n - q * d;
  if (r < 0) --q;
  else if (r >= d) ++q;
  return static_cast<int>(q);
}

struct Slice {
  int lo, hi;  // this workgroup's items [lo, hi) of the list
  int T, P;    // list length, workgroups sharing it
  int base;    // global FC1 block / FC2 unit of the list's first item
};

// List h: 0 = FC1(A), 1 = FC1(B), 2 = FC2(A), 3 = FC2(B); slices of near-equal length.
// Computed per lane (h may differ between lanes: fill_slices takes one list per lane);
// the kernel reads the results through the slice table (slice_at), as scalars.
__device__ __forceinline__ Slice make_slice(const ExpArgs& a, int n_chunks, int h) {
  const int cA = (n_chunks + 1) / 2;
  const int c_lo = (h & 1) ? cA : 0, c_hi = (h & 1) ? n_chunks : cA;
  const int per_chunk = h < 2 ? a.HB : a.U2;
  const int per = h < 2 ? a.HB * a.NSP : a.U2;
  const int G = static_cast<int>(gridDim.x), p = static_cast<int>(blockIdx.x);
  Slice s;
  s.T = (c_hi - c_lo) * per;
  s.base = c_lo * per_chunk;
  s.P = s.T < G ? s.T : G;
  if (h < 2 && a.qmin > 0 && s.T > 0) {
    // decode form: FC1 slices of at least qmin items, so a hidden block has at most
    // four owners (qmin = ceil(NSP / 3))
    const int q = s.T / a.qmin;
    s.P = q < 1 ? 1 : (q < s.P ? q : s.P);
  }
  s.lo = p < s.P ? div_floor(static_cast<int64_t>(p) * s.T, s.P) : 0;
  s.hi = p < s.P ? div_floor(static_cast<int64_t>(p + 1) * s.T, s.P) : 0;
  return s;
}

// Chunks that the workgroup's FC2 slice S spans: [first, first + count).
__device__ __forceinline__ int fc2_span(const ExpArgs& a, const Slice& S, int& first) {
  first = (S.base + S.lo) / a.U2;
  return S.hi > S.lo ? (S.base + S.hi - 1) / a.U2 - first + 1 : 0;
}

// The workgroup's four slices, computed once (threads 0-3, once the group list is in
// LDS) into the slice table: per list {lo, hi, T, P, base, FC2 span first / count, group
// of the chunk of the slice's first item}.  Readers take them with two LDS loads
// instead of the divisions.
struct SliceExtra {
  int span_first, span_count, g0;
};
__device__ __forceinline__ void fill_slices(const ExpArgs& a, const LdsMap& m, int n_groups, int n_chunks) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int h = threadIdx.x;
  if (h >= 4) return;
  const Slice S = make_slice(a, n_chunks, h);
  int first = 0, cnt = 0, g0 = 0;
  if (h >= 2) cnt = fc2_span(a, S, first);
  // group of the chunk holding the slice's first item (largest g with chunk0[g] <= c)
  const int per_chunk = h < 2 ? a.HB : a.U2, per_item = h < 2 ? a.NSP : 1;
  const int c = S.hi > S.lo ? (S.base + S.lo / per_item) / per_chunk : 0;
  const int* chunk0 = reinterpret_cast<const int*>(smem + m.chunk0);
  int lo = 0, hi = n_groups - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (chunk0[mid] <= c) lo = mid; else hi = mid - 1;
  }
  g0 = lo;
  int4* t = reinterpret_cast<int4*>(smem + m.slt + 32 * h);
  t[0] = make_int4(S.lo, S.hi, S.T, S.P);
  t[1] = make_int4(S.base, first, cnt, g0);
}
__device__ __forceinline__ Slice slice_at(const LdsMap& m, uint32_t lb, int h, SliceExtra* x = nullptr) {
  uint4 u, v;
  asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:16\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(u), "=&v"(v)
               : "v"(lb + m.slt + 32 * h)
               : "memory");
  Slice S;
  S.lo = __builtin_amdgcn_readfirstlane(static_cast<int>(u.x));
  S.hi = __builtin_amdgcn_readfirstlane(static_cast<int>(u.y));
  S.T = __builtin_amdgcn_readfirstlane(static_cast<int>(u.z));
  S.P = __builtin_amdgcn_readfirstlane(static_cast<int>(u.w));
  S.base = __builtin_amdgcn_readfirstlane(static_cast<int>(v.x));
  if (x) {
    x->span_first = __builtin_amdgcn_readfirstlane(static_cast<int>(v.y));
    x->span_count = __builtin_amdgcn_readfirstlane(static_cast<int>(v.z));
    x->g0 = __builtin_amdgcn_readfirstlane(static_cast<int>(v.w));
  }
  return S;
}

// Decode form: the partial-sum slots (512 tagged pairs each) of FC1 list h.  A slice of
// at most ceil(T/P) items touches at most (ceil(T/P) - 1) / NSP + 2 hidden blocks, so
// workgroup p's slots of list h are p * SPW_h + (local block); list 1's follow list 0's.
__device__ __forceinline__ int dec_spw(const Slice& S, int NSP) {
  return S.P > 0 ? ((S.T + S.P - 1) / S.P - 1) / NSP + 2 : 0;
}
// Slot of workgroup p's share of list-local FC1 block bl of list h (S = that list).
__device__ __forceinline__ uint32_t dec_slot(const ExpArgs& a, const Slice& S0, int h, const Slice& S, int p,
                                              int bl) {
  const uint32_t off = h == 1 ? static_cast<uint32_t>(S0.P * dec_spw(S0, a.NSP)) : 0u;
  const int lo = div_floor(static_cast<int64_t>(p) * S.T, S.P);
  return off + static_cast<uint32_t>(p * dec_spw(S, a.NSP) + (bl - lo / a.NSP));
}
// Owner of item x of a list of T items split over P slices: ceil((x + 1) P / T) - 1.
__device__ __forceinline__ int slice_owner(int x, int T, int P) {
  return div_floor(static_cast<int64_t>(x + 1) * P + T - 1, T) - 1;
}

// One wave's walk over its items: FC1 steps s_lo + w, s_lo + w + 4, ... of each block
// of the slice, then FC2 units lo + w, lo + w + 4, ...  Besides the position it tracks
// the item's chunk, its place in the chunk and the chunk's group, incrementally.
struct Cursor {
  int h;              // list 0..3; 4 = done; -1 = not started
  int lo, hi, base;   // the list's slice
  int b;              // FC1: block of the list; FC2: item of the list
  int s, s_hi;        // FC1: step pair in the block, end of the slice in the block
  int gidx;           // global block / unit of the item
  int chunk, j;       // its chunk, and hidden block (FC1) / output tile (FC2) in the chunk
  int seq0, cfirst;   // FC2: index of the list's first chunk in the workgroup's chunk sequence
  GroupInfo gi;       // the chunk's group
  int xrow, xsrow;    // FC1, per lane: offsets of its column's x codes (+ its K quarter) and scales
};

// Per lane: plan offsets of the x codes (+ the lane's K quarter) and x scales of the
// column the lane holds in the chunk (group gi, tile gi.cc); -1 for a padded column,
// whose loads then fall outside the plan buffer and bring zeros without touching memory.
__device__ __forceinline__ void x_rows(const ExpArgs& a, const LdsMap& m, uint32_t lb, const GroupInfo& gi,
                                       int& xrow, int& xsrow) {
  const int l = threadIdx.x & 63;
  const int pair = column_pair(m, lb, gi, gi.cc * 16 + (l & 15));
  const int t = pair >= 0 ? pair / a.K : 0;
  xrow = pair >= 0 ? t * a.D + 16 * (l >> 4) : -1;
  xsrow = pair >= 0 ? static_cast<int>(a.plan_bytes / 33u * 32u) + t * (a.D / 32) : -1;
}

template <bool DEC>
__device__ __forceinline__ void cursor_next(const ExpArgs& a, const LdsMap& m, uint32_t lb, int n_groups,
                                            int n_chunks, Cursor& c) {
  const int w = wave_id();
  if (c.h < 2) {
    c.s += 4;
    if (c.s < c.s_hi) return;  // same block
    c.b += 1;
  } else {
    c.b += 4;
  }
  bool fresh = false;
  for (;;) {
    if (c.h >= 0 && c.h < 2) {
      const int bs = c.b * a.NSP;
      if (bs < c.hi) {
        const int s_lo = c.lo > bs ? c.lo - bs : 0;
        const int s_hi = c.hi - bs < a.NSP ? c.hi - bs : a.NSP;
        if (s_hi - s_lo > w) {
          c.s = s_lo + w;
          c.s_hi = s_hi;
          break;
        }
        c.b += 1;
        continue;
      }
    } else if (c.h >= 2 && c.h < 4) {
      if (c.b < c.hi) break;
    }
    if (c.h >= 3) {
      c.h = 4;
      return;
    }
    ++c.h;
    SliceExtra sx;
    const Slice sl = slice_at(m, lb, c.h, &sx);
    c.lo = sl.lo;
    c.hi = sl.hi;
    c.base = sl.base;
    c.b = c.h < 2 ? c.lo / a.NSP : c.lo + w;
    c.gi.g = sx.g0;  // group of the slice's first chunk: the scan below starts there
    if (c.h >= 2) {
      c.cfirst = sx.span_first;
      c.seq0 = 0;
      if (c.h == 3) {
        SliceExtra s2;
        slice_at(m, lb, 2, &s2);
        c.seq0 = s2.span_count;
      }
    }
    fresh = true;
  }
  const int per_chunk = c.h < 2 ? a.HB : a.U2;
  const int gidx = c.base + c.b;
  bool moved = fresh;
  if (fresh) {
    c.chunk = gidx / per_chunk;
    c.j = gidx - c.chunk * per_chunk;
    int g = c.gi.g;
    while (g + 1 < n_groups && c.chunk >= lds_uni(lb + m.chunk0 + 4 * g + 4)) ++g;
    GroupInfo gi = group_at(m, lb, g);
    gi.cc = c.chunk - gi.c0;
    c.gi = gi;
  } else {
    int j = c.j + gidx - c.gidx, chunk = c.chunk;
    while (j >= per_chunk) {
      j -= per_chunk;
      ++chunk;
    }
    c.j = j;
    if (chunk != c.chunk) {
      int g = c.gi.g;
      while (chunk >= lds_uni(lb + m.chunk0 + 4 * g + 4)) ++g;
      GroupInfo gi = group_at(m, lb, g);
      gi.cc = chunk - gi.c0;
      c.gi = gi;
      c.chunk = chunk;
      moved = true;
    }
  }
  if (!DEC && moved && c.h < 2) x_rows(a, m, lb, c.gi, c.xrow, c.xsrow);
  c.gidx = gidx;
}

// ------------------------------------------------------------ the item stream
// A wave's item k lives in ring slot k % R of the wave.  FC1 item (two K steps s0, s0+1
// of one hidden block): [A: 2 x four 1 KB FP4 row tiles][A scales: 2 x one word per
// lane][x: 2 x the 2 KB FP8 B operand][x scales: 2 x one word per lane].  FC2 item (T2
// output tiles): [A: T2 x NS2 1 KB FP4 tiles] ... [A scales: T2 x one word per lane].
// Every item issues the same number L of DMA instructions (FC2 items and the dummies
// past the end pad with redundant word loads into unused bytes of their slot), so "the
// oldest of R items has landed" is always s_waitcnt vmcnt((R-1)*L).  The item's 16-byte
// record goes to LDS when it is issued.
constexpr uint32_t kSlotAS = 8192, kSlotX = 8704, kSlotXS = 12800;

__device__ __forceinline__ void lds_st16_async(uint32_t addr, uint4 v) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  const v4u x = {v.x, v.y, v.z, v.w};
  asm volatile("ds_write_b128 %0, %1" : : "v"(addr), "v"(x) : "memory");
}

template <int NS2, int R, bool DEC>
__device__ __forceinline__ void issue_item(const ExpArgs& a, const LdsMap& m, uint32_t lb, const Cursor& c, int k,
                                           __amdgpu_buffer_rsrc_t xr) {
  using G = Geo<1, R, NS2, DEC>;
  constexpr int T2 = Fc2Tiles<NS2>::T2;
  const int l = threadIdx.x & 63, w = wave_id();
  const int slot = k % R;
  const uint32_t so = m.ring + (w * R + slot) * G::SLOT;  // offset from the LDS base
  uint4 meta = make_uint4(2u, 0u, 0u, 0u);                   // 2: dummy
  int done = 0;
  // an expert index outside [0, E) can only come from a broken invariant: issue nothing
  // from it (the item turns into a dummy) and flag it, rather than load out of bounds
  const bool sane = c.gi.e >= 0 && c.gi.e < a.E;
  if (c.h < 4 && !sane && l == 0) __hip_atomic_fetch_or(a.err, 4, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (c.h < 2 && sane) {
    const int s0 = 2 * c.s;
    const int64_t step = static_cast<int64_t>(c.gi.e * a.HB + c.j) * a.NS1 + s0;
    const uint8_t* wb = a.w13p + step * 4096 + l * 16;
#pragma unroll
    for (int i = 0; i < 8; ++i) dma16(wb + i * 1024, so + i * 1024);
    const uint8_t* sb = a.s13p + step * 256 + l * 4;
    dma4(sb, so + kSlotAS);
    dma4(sb + 256, so + kSlotAS + 256);
    if constexpr (DEC) {
      // x is in LDS: the record names the chunk and the step pair instead
      meta = make_uint4(0u, static_cast<uint32_t>(c.gidx), static_cast<uint32_t>(c.chunk),
                        static_cast<uint32_t>(c.s));
      done = 10;
    } else {
      const bool live = c.xrow >= 0;
      const uint32_t xo = live ? static_cast<uint32_t>(c.xrow + s0 * 128) : kOutside;
#pragma unroll
      for (int i = 0; i < 4; ++i) bdma16(xr, live ? xo + i * 64 : kOutside, so + kSlotX + i * 1024);
      const uint32_t xso = live ? static_cast<uint32_t>(c.xsrow + 4 * s0) : kOutside;
      bdma4(xr, xso, so + kSlotXS);
      bdma4(xr, live ? xso + 4 : kOutside, so + kSlotXS + 256);
      meta = make_uint4(0u, static_cast<uint32_t>(c.gidx), 0u, 0u);
      done = G::L;
    }
  } else if (c.h < 4 && sane) {
    const int64_t tile = static_cast<int64_t>(c.gi.e) * (a.D / 16) + c.j * T2;
    const uint8_t* wb = a.w2p + tile * NS2 * 1024 + l * 16;
#pragma unroll
    for (int i = 0; i < T2 * NS2; ++i) dma16(wb + i * 1024, so + i * 1024);
    const uint8_t* sb = a.s2p + tile * 256 + l * 4;
#pragma unroll
    for (int t = 0; t < T2; ++t) dma4(sb + t * 256, so + kSlotAS + t * 256);
    meta = make_uint4(1u, static_cast<uint32_t>(c.chunk), static_cast<uint32_t>(c.j),
                      static_cast<uint32_t>(c.seq0 + c.chunk - c.cfirst));
    done = T2 * NS2 + T2;
  }
  for (int i = done; i < G::L; ++i) bdma4(xr, kOutside, so + G::PAD);
  if (l == 0) lds_st16_async(lb + m.meta + (w * R + slot) * 16, meta);
}

// ------------------------------------------------------------ item operand reads
// Every read of an item's operands is one asm block with a single LDS wait (the DMA
// stream must not be drained by the compiler's conservative waits).

// FC1 item: A = two K steps x four row tiles (a[step*4 + rt] at pa + 4096 step + 1024 rt),
// A scale words (as[step] at pq + 8192 + 256 step), x halves (x[step*2 + half] at
// pa + 8704 + 2048 step + 1024 half) and x scale words (xs[step] at pq + 12800 + 256 step).
struct Fc1Ops {
  uint4 a[8], x[4];
  uint32_t as[2], xs[2];
};
__device__ __forceinline__ void fc1_read(uint32_t pa, uint32_t pq, Fc1Ops& o) {
  asm volatile(
      "ds_read_b128 %0, %16 offset:0\n\t"
      "ds_read_b128 %1, %16 offset:1024\n\t"
      "ds_read_b128 %2, %16 offset:2048\n\t"
      "ds_read_b128 %3, %16 offset:3072\n\t"
      "ds_read_b128 %4, %16 offset:4096\n\t"
      "ds_read_b128 %5, %16 offset:5120\n\t"
      "ds_read_b128 %6, %16 offset:6144\n\t"
      "ds_read_b128 %7, %16 offset:7168\n\t"
      "ds_read_b32 %12, %17 offset:8192\n\t"
      "ds_read_b32 %13, %17 offset:8448\n\t"
      "ds_read_b128 %8, %16 offset:8704\n\t"
      "ds_read_b128 %9, %16 offset:9728\n\t"
      "ds_read_b128 %10, %16 offset:10752\n\t"
      "ds_read_b128 %11, %16 offset:11776\n\t"
      "ds_read_b32 %14, %17 offset:12800\n\t"
      "ds_read_b32 %15, %17 offset:13056\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o.a[0]), "=&v"(o.a[1]), "=&v"(o.a[2]), "=&v"(o.a[3]), "=&v"(o.a[4]), "=&v"(o.a[5]), "=&v"(o.a[6]), "=&v"(o.a[7]), "=&v"(o.x[0]), "=&v"(o.x[1]), "=&v"(o.x[2]), "=&v"(o.x[3]), "=&v"(o.as[0]), "=&v"(o.as[1]), "=&v"(o.xs[0]), "=&v"(o.xs[1])
      : "v"(pa), "v"(pq)
      : "memory");
}

// Decode form FC1 item: A and its scale words from the slot (as fc1_read), the x operand
// from the LDS plan: px = the column's codes at the item's first K step (+ 16 per lane
// group), halves at +0/+64 (step 0) and +128/+192 (step 1); pxs = its scale words.
__device__ __forceinline__ void fc1_read_dec(uint32_t pa, uint32_t pq, uint32_t px, uint32_t pxs, Fc1Ops& o) {
  asm volatile(
      "ds_read_b128 %0, %16 offset:0\n\t"
      "ds_read_b128 %1, %16 offset:1024\n\t"
      "ds_read_b128 %2, %16 offset:2048\n\t"
      "ds_read_b128 %3, %16 offset:3072\n\t"
      "ds_read_b128 %4, %16 offset:4096\n\t"
      "ds_read_b128 %5, %16 offset:5120\n\t"
      "ds_read_b128 %6, %16 offset:6144\n\t"
      "ds_read_b128 %7, %16 offset:7168\n\t"
      "ds_read_b32 %12, %17 offset:8192\n\t"
      "ds_read_b32 %13, %17 offset:8448\n\t"
      "ds_read_b128 %8, %18 offset:0\n\t"
      "ds_read_b128 %9, %18 offset:64\n\t"
      "ds_read_b128 %10, %18 offset:128\n\t"
      "ds_read_b128 %11, %18 offset:192\n\t"
      "ds_read_b32 %14, %19 offset:0\n\t"
      "ds_read_b32 %15, %19 offset:4\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o.a[0]), "=&v"(o.a[1]), "=&v"(o.a[2]), "=&v"(o.a[3]), "=&v"(o.a[4]), "=&v"(o.a[5]), "=&v"(o.a[6]), "=&v"(o.a[7]), "=&v"(o.x[0]), "=&v"(o.x[1]), "=&v"(o.x[2]), "=&v"(o.x[3]), "=&v"(o.as[0]), "=&v"(o.as[1]), "=&v"(o.xs[0]), "=&v"(o.xs[1])
      : "v"(pa), "v"(pq), "v"(px), "v"(pxs)
      : "memory");
}

// FC2: the hidden's B operand of a chunk column (per K step s: halves at pb + 128 s and
// + 64, scale word at ps + 4 s), read once per item.
template <int NS2>
struct HidOps {
  uint4 bl[NS2], bh[NS2];
  uint32_t bs[NS2];
};
template <int NS2>
__device__ __forceinline__ void hid_read(uint32_t pb, uint32_t ps, HidOps<NS2>& o);
// FC2 item: T2 output tiles of NS2 K steps each (a[t*NS2 + s] at pa + 1024 (t NS2 + s)),
// one A scale word per tile (as[t] at pq + 8192 + 256 t).
template <int NS2, int T2>
struct Fc2Ops {
  uint4 a[T2 * NS2];
  uint32_t as[T2];
};
template <int NS2, int T2>
__device__ __forceinline__ void fc2_read(uint32_t pa, uint32_t pq, Fc2Ops<NS2, T2>& o);

template <>
__device__ __forceinline__ void hid_read<1>(uint32_t pb, uint32_t ps, HidOps<1>& o) {
  asm volatile(
      "ds_read_b128 %0, %3 offset:0\n\t"
      "ds_read_b128 %1, %3 offset:64\n\t"
      "ds_read_b32 %2, %4 offset:0\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o.bl[0]), "=&v"(o.bh[0]), "=&v"(o.bs[0])
      : "v"(pb), "v"(ps)
      : "memory");
}

template <>
__device__ __forceinline__ void hid_read<2>(uint32_t pb, uint32_t ps, HidOps<2>& o) {
  asm volatile(
      "ds_read_b128 %0, %6 offset:0\n\t"
      "ds_read_b128 %1, %6 offset:64\n\t"
      "ds_read_b32 %2, %7 offset:0\n\t"
      "ds_read_b128 %3, %6 offset:128\n\t"
      "ds_read_b128 %4, %6 offset:192\n\t"
      "ds_read_b32 %5, %7 offset:4\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o.bl[0]), "=&v"(o.bh[0]), "=&v"(o.bs[0]), "=&v"(o.bl[1]), "=&v"(o.bh[1]), "=&v"(o.bs[1])
      : "v"(pb), "v"(ps)
      : "memory");
}

template <>
__device__ __forceinline__ void hid_read<3>(uint32_t pb, uint32_t ps, HidOps<3>& o) {
  asm volatile(
      "ds_read_b128 %0, %9 offset:0\n\t"
      "ds_read_b128 %1, %9 offset:64\n\t"
      "ds_read_b32 %2, %10 offset:0\n\t"
      "ds_read_b128 %3, %9 offset:128\n\t"
      "ds_read_b128 %4, %9 offset:192\n\t"
      "ds_read_b32 %5, %10 offset:4\n\t"
      "ds_read_b128 %6, %9 offset:256\n\t"
      "ds_read_b128 %7, %9 offset:320\n\t"
      "ds_read_b32 %8, %10 offset:8\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o.bl[0]), "=&v"(o.bh[0]), "=&v"(o.bs[0]), "=&v"(o.bl[1]), "=&v"(o.bh[1]), "=&v"(o.bs[1]), "=&v"(o.bl[2]), "=&v"(o.bh[2]), "=&v"(o.bs[2])
      : "v"(pb), "v"(ps)
      : "memory");
}

template <>
__device__ __forceinline__ void hid_read<4>(uint32_t pb, uint32_t ps, HidOps<4>& o) {
  asm volatile(
      "ds_read_b128 %0, %12 offset:0\n\t"
      "ds_read_b128 %1, %12 offset:64\n\t"
      "ds_read_b32 %2, %13 offset:0\n\t"
      "ds_read_b128 %3, %12 offset:128\n\t"
      "ds_read_b128 %4, %12 offset:192\n\t"
      "ds_read_b32 %5, %13 offset:4\n\t"
      "ds_read_b128 %6, %12 offset:256\n\t"
      "ds_read_b128 %7, %12 offset:320\n\t"
      "ds_read_b32 %8, %13 offset:8\n\t"
      "ds_read_b128 %9, %12 offset:384\n\t"
      "ds_read_b128 %10, %12 offset:448\n\t"
      "ds_read_b32 %11, %13 offset:12\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o.bl[0]), "=&v"(o.bh[0]), "=&v"(o.bs[0]), "=&v"(o.bl[1]), "=&v"(o.bh[1]), "=&v"(o.bs[1]), "=&v"(o.bl[2]), "=&v"(o.bh[2]), "=&v"(o.bs[2]), "=&v"(o.bl[3]), "=&v"(o.bh[3]), "=&v"(o.bs[3])
      : "v"(pb), "v"(ps)
      : "memory");
}

template <>
__device__ __forceinline__ void fc2_read<1, 8>(uint32_t pa, uint32_t pq, Fc2Ops<1, 8>& o) {
  asm volatile(
      "ds_read_b128 %0, %16 offset:0\n\t"
      "ds_read_b128 %1, %16 offset:1024\n\t"
      "ds_read_b128 %2, %16 offset:2048\n\t"
      "ds_read_b128 %3, %16 offset:3072\n\t"
      "ds_read_b128 %4, %16 offset:4096\n\t"
      "ds_read_b128 %5, %16 offset:5120\n\t"
      "ds_read_b128 %6, %16 offset:6144\n\t"
      "ds_read_b128 %7, %16 offset:7168\n\t"
      "ds_read_b32 %8, %17 offset:8192\n\t"
      "ds_read_b32 %9, %17 offset:8448\n\t"
      "ds_read_b32 %10, %17 offset:8704\n\t"
      "ds_read_b32 %11, %17 offset:8960\n\t"
      "ds_read_b32 %12, %17 offset:9216\n\t"
      "ds_read_b32 %13, %17 offset:9472\n\t"
      "ds_read_b32 %14, %17 offset:9728\n\t"
      "ds_read_b32 %15, %17 offset:9984\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o.a[0]), "=&v"(o.a[1]), "=&v"(o.a[2]), "=&v"(o.a[3]), "=&v"(o.a[4]), "=&v"(o.a[5]), "=&v"(o.a[6]), "=&v"(o.a[7]), "=&v"(o.as[0]), "=&v"(o.as[1]), "=&v"(o.as[2]), "=&v"(o.as[3]), "=&v"(o.as[4]), "=&v"(o.as[5]), "=&v"(o.as[6]), "=&v"(o.as[7])
      : "v"(pa), "v"(pq)
      : "memory");
}

template <>
__device__ __forceinline__ void fc2_read<2, 4>(uint32_t pa, uint32_t pq, Fc2Ops<2, 4>& o) {
  asm volatile(
      "ds_read_b128 %0, %12 offset:0\n\t"
      "ds_read_b128 %1, %12 offset:1024\n\t"
      "ds_read_b128 %2, %12 offset:2048\n\t"
      "ds_read_b128 %3, %12 offset:3072\n\t"
      "ds_read_b128 %4, %12 offset:4096\n\t"
      "ds_read_b128 %5, %12 offset:5120\n\t"
      "ds_read_b128 %6, %12 offset:6144\n\t"
      "ds_read_b128 %7, %12 offset:7168\n\t"
      "ds_read_b32 %8, %13 offset:8192\n\t"
      "ds_read_b32 %9, %13 offset:8448\n\t"
      "ds_read_b32 %10, %13 offset:8704\n\t"
      "ds_read_b32 %11, %13 offset:8960\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o.a[0]), "=&v"(o.a[1]), "=&v"(o.a[2]), "=&v"(o.a[3]), "=&v"(o.a[4]), "=&v"(o.a[5]), "=&v"(o.a[6]), "=&v"(o.a[7]), "=&v"(o.as[0]), "=&v"(o.as[1]), "=&v"(o.as[2]), "=&v"(o.as[3])
      : "v"(pa), "v"(pq)
      : "memory");
}

template <>
__device__ __forceinline__ void fc2_read<3, 2>(uint32_t pa, uint32_t pq, Fc2Ops<3, 2>& o) {
  asm volatile(
      "ds_read_b128 %0, %8 offset:0\n\t"
      "ds_read_b128 %1, %8 offset:1024\n\t"
      "ds_read_b128 %2, %8 offset:2048\n\t"
      "ds_read_b128 %3, %8 offset:3072\n\t"
      "ds_read_b128 %4, %8 offset:4096\n\t"
      "ds_read_b128 %5, %8 offset:5120\n\t"
      "ds_read_b32 %6, %9 offset:8192\n\t"
      "ds_read_b32 %7, %9 offset:8448\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o.a[0]), "=&v"(o.a[1]), "=&v"(o.a[2]), "=&v"(o.a[3]), "=&v"(o.a[4]), "=&v"(o.a[5]), "=&v"(o.as[0]), "=&v"(o.as[1])
      : "v"(pa), "v"(pq)
      : "memory");
}

template <>
__device__ __forceinline__ void fc2_read<4, 2>(uint32_t pa, uint32_t pq, Fc2Ops<4, 2>& o) {
  asm volatile(
      "ds_read_b128 %0, %10 offset:0\n\t"
      "ds_read_b128 %1, %10 offset:1024\n\t"
      "ds_read_b128 %2, %10 offset:2048\n\t"
      "ds_read_b128 %3, %10 offset:3072\n\t"
      "ds_read_b128 %4, %10 offset:4096\n\t"
      "ds_read_b128 %5, %10 offset:5120\n\t"
      "ds_read_b128 %6, %10 offset:6144\n\t"
      "ds_read_b128 %7, %10 offset:7168\n\t"
      "ds_read_b32 %8, %11 offset:8192\n\t"
      "ds_read_b32 %9, %11 offset:8448\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o.a[0]), "=&v"(o.a[1]), "=&v"(o.a[2]), "=&v"(o.a[3]), "=&v"(o.a[4]), "=&v"(o.a[5]), "=&v"(o.a[6]), "=&v"(o.a[7]), "=&v"(o.as[0]), "=&v"(o.as[1])
      : "v"(pa), "v"(pq)
      : "memory");
}

// The control wave's end of FC1 block lbk of list `half` (the experts page's
// ExpertsKernel.partials and store_hidden).  acc holds the block's sums over this
// workgroup's steps.  A block inside the slice is finished at once.  A block split over
// several workgroups' slices is finished by the owner of its first step, for which it
// is the slice's last block: the others (for which it is their first block) file their
// partial sums and count in without waiting, and the finisher adds them in slice order.
// No workgroup ever waits for a block that a wait of its own delays.  Finishing =
// SwiGLU + MXFP8 of the hidden block for every column tile of the chunk, then its
// flag, tagged with the call number.
template <int NT>
__device__ __forceinline__ void control_block(const ExpArgs& a, const LdsMap& m, uint32_t lb, int n_groups,
                                              const Slice& li, int half, int lbk, v4f (&acc)[4][NT],
                                              uint32_t gen) {
  static_assert(NT == 1, "one column tile per block");
  const int l = threadIdx.x & 63;
  const int NS1 = a.NSP, HB = a.HB;  // block length in FC1 items (step pairs)
  const int p = blockIdx.x;
  const int b = li.base + lbk;  // global block
  const int bs = lbk * NS1;
  const int chunk = b / HB, j = b - chunk * HB;
  const GroupInfo gi = group_of(m, lb, n_groups, chunk);
  // the lane's column holds a route (padded columns are neither filed nor summed: every
  // FC2 output column depends on its own hidden column only, and padded rows are never
  // stored)
  const int pair = column_pair(m, lb, gi, gi.cc * 16 + (l & 15));
  const bool live = pair >= 0;
  if (li.lo > bs) {
    // contributor: file the partial sums (device-coherent, two floats per store), then
    // count in
    float* slot = a.partials + (static_cast<int64_t>(p) * 2 + half) * NT * 1024 + l * 4;
    if (live)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int r = 0; r < 4; r += 2)
          st_dev_u64(slot + rt * 256 + r, (static_cast<uint64_t>(__float_as_uint(acc[rt][0][r + 1])) << 32) |
                                              __float_as_uint(acc[rt][0][r]));
    wait_stores();
    if (l == 0) __hip_atomic_fetch_add(a.arrive + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  if (bs + NS1 > li.hi) {
    // finisher: the block's other steps belong to slices p+1 .. pb (slice p holds steps
    // [floor(pT/P), floor((p+1)T/P)); the owner of step x is ceil((x+1)P/T) - 1)
    const int T = li.T, P = li.P;
    const int pb = div_floor(static_cast<int64_t>(bs + NS1) * P + T - 1, T) - 1;
    const uint32_t want = static_cast<uint32_t>(pb - p);
    #pragma unroll 1
    for (uint32_t spins = 0;; ++spins) {
      if (ld_dev_u32(a.arrive + b) == want) break;
      if (poll_expired(spins, a.err)) {
        if (l == 0) __hip_atomic_fetch_or(a.err, 4, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    compiler_fence();
    if (l == 0) st_dev_u32(a.arrive + b, 0u);  // re-arm for the next call
    // up to four contributors' partials in flight at once, added in slice order
    for (int pp0 = p + 1; pp0 <= pb; pp0 += 4) {
      uint64_t v[4][NT * 8];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (pp0 + u > pb || !live) continue;
        const float* src = a.partials + (static_cast<int64_t>(pp0 + u) * 2 + half) * NT * 1024 + l * 4;
#pragma unroll
        for (int i = 0; i < NT * 4; ++i) {
          v[u][2 * i] = ld_dev_u64(src + i * 256);
          v[u][2 * i + 1] = ld_dev_u64(src + i * 256 + 2);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (pp0 + u > pb || !live) continue;
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) {
            const uint64_t v0 = v[u][2 * (n * 4 + rt)], v1 = v[u][2 * (n * 4 + rt) + 1];
            acc[rt][n][0] += __uint_as_float(static_cast<uint32_t>(v0));
            acc[rt][n][1] += __uint_as_float(static_cast<uint32_t>(v0 >> 32));
            acc[rt][n][2] += __uint_as_float(static_cast<uint32_t>(v1));
            acc[rt][n][3] += __uint_as_float(static_cast<uint32_t>(v1 >> 32));
          }
      }
    }
  }
  {
    const v4f tot[4] = {acc[0][0], acc[1][0], acc[2][0], acc[3][0]};
    hidden_epilogue(a, tot, j, gi.tile0 + gi.cc, pair);
  }
  // Publish: the block's codes and scales are stored (sc1) before its flag.
  wait_stores();
  if (l == 0) st_dev_u32(a.flags + b, gen + 1);
}

// Wait until the HB hidden blocks of a chunk carry this call's tag.  Bounded (seconds)
// so that a broken invariant can never hang the GPU: it then flags the unit table
// header (bit 2) and goes on with whatever is there.
__device__ __forceinline__ void wait_chunk(const ExpArgs& a, int chunk, uint32_t gen) {
  const int l = threadIdx.x & 63;
  const uint32_t want = gen + 1;
  const uint32_t* f = a.flags + static_cast<int64_t>(chunk) * a.HB;
  #pragma unroll 1
  for (uint32_t spins = 0;; ++spins) {
    bool ok = true;
    for (int i = l; i < a.HB; i += 64) ok = ok && ld_dev_u32(f + i) == want;
    if (__all(ok)) break;
    if (poll_expired(spins, a.err)) {
      if (l == 0) __hip_atomic_fetch_or(a.err, 4, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  compiler_fence();
}

// The control wave's copy of one FC2 chunk's hidden (codes and scales of its NT column
// tiles, as FC1 published them) into hidden buffer `buf`.  Per tile: 16 columns x IP
// code bytes (IP = 128 * NS2, contiguous: 2 * NS2 16-byte pieces per lane) and 16 x
// IP/32 scale bytes (one word per lane), all loaded in one batch.
template <int NT, int NS2>
__device__ __forceinline__ void control_hidden(const ExpArgs& a, const LdsMap& m, uint32_t lb, int n_groups,
                                               int chunk, uint32_t buf) {
  const int l = threadIdx.x & 63;
  const GroupInfo gi = group_of(m, lb, n_groups, chunk);
  constexpr int IP = 128 * NS2, PER_COL = IP / 16, SW = IP / 32;
  const uint32_t hb = lb + m.hid + buf * m.hid_bytes;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int t = gi.cc * NT + n;
    if (t >= gi.ntiles) continue;
    const int64_t gcol0 = static_cast<int64_t>(gi.tile0 + t) * 16;
    const uint8_t* src = a.hcodes + gcol0 * IP;
    const uint8_t* ssrc = a.hscales + gcol0 * SW;
    uint64_t v[2 * NS2][2];
#pragma unroll
    for (int u = 0; u < 2 * NS2; ++u) {
      const int q = u * 64 + l;
      v[u][0] = ld_dev_u64(src + q * 16);
      v[u][1] = ld_dev_u64(src + q * 16 + 8);
    }
    const uint32_t sw = l < 4 * SW ? ld_dev_u32(ssrc + l * 4) : 0u;
#pragma unroll
    for (int u = 0; u < 2 * NS2; ++u) {
      const int q = u * 64 + l, col = q / PER_COL, off = (q - col * PER_COL) * 16;
      lds_st16(hb + (n * 16 + col) * m.hs + off,
               make_uint4(static_cast<uint32_t>(v[u][0]), static_cast<uint32_t>(v[u][0] >> 32),
                          static_cast<uint32_t>(v[u][1]), static_cast<uint32_t>(v[u][1] >> 32)));
    }
    if (l < 4 * SW) lds_st4(hb + NT * 16 * m.hs + n * 16 * SW + l * 4, sw);
  }
}

// ------------------------------------------------------------ decode form exchange
// FC1 block sums cross workgroups as call-tagged (float bits, call + 1) pairs that the
// FC2 side reduces itself: one store and one load between a block's last FC1 step and
// FC2, where a finished-block scheme needs a count, a finisher's loads, the hidden's
// stores and a flag.

__device__ __forceinline__ void lds_st1(uint32_t addr, uint32_t v) {
  asm volatile("ds_write_b8 %0, %1" : : "v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_st4_nw(uint32_t addr, uint32_t v) {
  asm volatile("ds_write_b32 %0, %1" : : "v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_settle() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Real token columns of a decode-form group (its one unit's non-padding entries).
__device__ __forceinline__ int unit_cols(const LdsMap& m, uint32_t lb, const GroupInfo& gi) {
  const int l = threadIdx.x & 63;
  const uint32_t v = lds_ld2(lb + m.urows + (gi.unit0 * 8 + (l & 7)) * 2);
  return __popcll(__ballot(l < 8 && v != 0xffffu));
}

// File the workgroup's sum of list-local FC1 block lbk of list h (the four streaming
// waves' sums in hand-over slot q & 1, added in wave order): lane l = block row l (gate
// rows 0-31, up rows 32-63), one 64-pair run per real column.  No wait.
__device__ __forceinline__ void dec_publish(const ExpArgs& a, const LdsMap& m, uint32_t lb, int n_groups,
                                            int n_chunks, const Slice& S, int h, int lbk, int q, uint32_t gen) {
  const int l = threadIdx.x & 63;
  const int chunk = (S.base + lbk) / a.HB;
  const GroupInfo gi = group_of(m, lb, n_groups, chunk);
  const int ncols = unit_cols(m, lb, gi);
  uint64_t* dst = a.dpart + static_cast<size_t>(dec_slot(a, slice_at(m, lb, 0), h, S, blockIdx.x, lbk)) * 512 + l;
  // element (row l, column c) of tile rt = l / 16 sits in lane 16 ((l % 16) / 4) + c,
  // register l % 4 of the MFMA result
  const int rt = l >> 4, rr = l & 15;
  const uint32_t src = lb + m.red + ((q & 1) * kStream * 4 + rt) * 1024 + 256 * (rr >> 2) + 4 * (rr & 3);
  const uint64_t tag = static_cast<uint64_t>(gen + 1) << 32;
  static_assert(kStream == 4, "four streaming waves' sums");
  for (int c = 0; c < ncols; ++c) {
    uint32_t x0, x1, x2, x3;
    lds_ld4x4<0, 4096>(src + 16 * c, x0, x1, x2, x3);
    const float v = ((__uint_as_float(x0) + __uint_as_float(x1)) + __uint_as_float(x2)) + __uint_as_float(x3);
    st_dev_u64(dst + 64 * c, tag | __float_as_uint(v));
  }
}

// The hidden of FC2 chunk `chunk` (one expert, up to 8 token columns) into hidden buffer
// buf, from the tagged FC1 partials: per hidden block j and column c, the owners' sums
// added in slice order, then SwiGLU and MXFP8 (experts page, store_hidden: FP32 hidden,
// one E8M0 exponent per 32 values; the arithmetic of hidden_epilogue).
// The partial pairs are taken in (block, column, owner) order, kRound per lane at a time:
// lane s works out where pair s of a round lives (from a per-chunk table in LDS) and
// whether it opens or closes a (block, column) sum; the loads take those addresses by
// lane broadcasts.  Before loading, it polls one probe pair per (block, owner) -- the last
// pair each owner stores; a round whose tags are not all this call's is loaded again
// (bounded).  Finished sums are staged in LDS and completed two at a time, one per
// half-wave.  The workgroup owning the chunk's first FC2 item writes the optional dump.
__device__ __forceinline__ void dec_hidden(const ExpArgs& a, const LdsMap& m, uint32_t lb, int n_groups,
                                           int n_chunks, int chunk, uint32_t buf, bool dump, uint32_t gen) {
  const int l = threadIdx.x & 63, half = l >> 5, hl = l & 31;
  const GroupInfo gi = group_of(m, lb, n_groups, chunk);
  const int ncols = unit_cols(m, lb, gi);
  const int HB = a.HB, NSP = a.NSP;
  const uint32_t want = gen + 1;
  // lane 4j + k: owner k (< 4) of hidden block j and its slot; the table: cum[16] (first
  // pair of block j in the chunk's order), nown[16], slot[64]
  const uint32_t tb = lb + m.scr + kRound * 256;
  int total;
  {
    const int h = chunk < (n_chunks + 1) / 2 ? 0 : 1;
    const Slice S = slice_at(m, lb, h), S0 = slice_at(m, lb, 0);
    const int j = l >> 2, k = l & 3;
    int nown = 0;
    uint32_t sidx = 0;
    if (j < HB) {
      const int bl = chunk * HB + j - S.base;
      const int p0 = slice_owner(bl * NSP, S.T, S.P), p1 = slice_owner(bl * NSP + NSP - 1, S.T, S.P);
      nown = p1 - p0 + 1;
      if (k < nown) sidx = dec_slot(a, S0, h, S, p0 + k, bl);
    }
    const int v = k == 0 ? nown * ncols : 0;
    int inc = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(inc, d);
      if (l >= d) inc += o;
    }
    total = __builtin_amdgcn_readlane(inc, 63);
    if (k == 0 && j < 16) {
      lds_st4_nw(tb + 4 * j, static_cast<uint32_t>(j < HB ? inc - v : total));
      lds_st4_nw(tb + 64 + 4 * j, static_cast<uint32_t>(nown));
    }
    lds_st4_nw(tb + 128 + 4 * l, sidx);
    lds_settle();
    const bool probe = j < HB && k < nown;
    const uint64_t* pp = a.dpart + static_cast<size_t>(sidx) * 512 + 64 * (ncols - 1) + 63;
#pragma unroll 1
    for (uint32_t spins = 0;; ++spins) {
      const bool ok = !probe || static_cast<uint32_t>(ld_dev_u64(pp) >> 32) == want;
      if (__all(ok)) break;
      if (poll_expired(spins, a.err)) {
        if (l == 0) __hip_atomic_fetch_or(a.err, 4, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(8);
    }
  }
  const uint32_t hb = lb + m.hid + buf * m.hid_bytes;
  int fj = 0, fc = 0;  // first unfinished (block, column)
  float sum = 0.0f;
#pragma unroll 1
  for (int done = 0; done < total; done += kRound) {
    const int nb = total - done < kRound ? total - done : kRound;
    // lane s: pair done + s -> block j (the last with cum[j] <= f), column, owner
    uint32_t poff = 0;  // pair offset of the lane's slot (global loads index a.dpart with it)
    bool first = false, last = false;
    {
      const int f = done + l;
      uint4 c4[4];
      asm volatile(
          "ds_read_b128 %0, %4 offset:0\n\t"
          "ds_read_b128 %1, %4 offset:16\n\t"
          "ds_read_b128 %2, %4 offset:32\n\t"
          "ds_read_b128 %3, %4 offset:48\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(c4[0]), "=&v"(c4[1]), "=&v"(c4[2]), "=&v"(c4[3])
          : "v"(tb)
          : "memory");
      int j = -1;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        j += (static_cast<int>(c4[q].x) <= f) + (static_cast<int>(c4[q].y) <= f) + (static_cast<int>(c4[q].z) <= f) +
             (static_cast<int>(c4[q].w) <= f);
      }
      j = j < HB - 1 ? j : HB - 1;  // blocks past HB carry cum = total
      if (l < nb) {
        const int cum = static_cast<int>(lds_ld4(tb + 4 * j));
        const int n = static_cast<int>(lds_ld4(tb + 64 + 4 * j));
        const int r = f - cum, c = r / n, k = r - c * n;
        const uint32_t sl = lds_ld4(tb + 128 + 4 * (4 * j + k));
        poff = sl * 512 + 64 * c;
        first = k == 0;
        last = k == n - 1;
      }
    }
    const uint64_t fm = __ballot(first), lm = __ballot(last);
    uint64_t v[kRound];
#pragma unroll 1
    for (uint32_t spins = 0;; ++spins) {
#pragma unroll
      for (int s = 0; s < kRound; ++s) {
        if (s < nb) {
          // slot s's pair offset from lane s; the load stays a global one (a generic one
          // would also count against the LDS counter, and the waits would serialize them)
          const uint32_t o = __builtin_amdgcn_readlane(poff, s);
          v[s] = ld_dev_u64(a.dpart + o + l);
        }
      }
      bool ok = true;
#pragma unroll
      for (int s = 0; s < kRound; ++s) ok = ok && (s >= nb || static_cast<uint32_t>(v[s] >> 32) == want);
      if (__all(ok)) break;
      if (poll_expired(spins, a.err)) {
        if (l == 0) __hip_atomic_fetch_or(a.err, 4, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(8);
    }
    // owners' sums in registers; each finished (block, column) sum goes to the staging area
    int nf = 0;
#pragma unroll
    for (int s = 0; s < kRound; ++s) {
      if (s < nb) {
        const float x = __uint_as_float(static_cast<uint32_t>(v[s]));
        sum = ((fm >> s) & 1) ? x : sum + x;
        if ((lm >> s) & 1) {
          lds_st4_nw(lb + m.scr + nf * 256 + l * 4, __float_as_uint(sum));
          ++nf;
        }
      }
    }
    lds_settle();
    // complete the finished sums two at a time: half-wave 0 takes (fj, fc), half-wave 1
    // the next; lane hl of a half is hidden row 32 fj + hl (its gate and up rows sit in
    // lanes hl and hl + 32 of the staged sums)
#pragma unroll 1
    for (int f = 0; f < nf; f += 2) {
      const bool two = f + 1 < nf;
      const float sA = __uint_as_float(lds_ld4(lb + m.scr + f * 256 + l * 4));
      const float sB = two ? __uint_as_float(lds_ld4(lb + m.scr + (f + 1) * 256 + l * 4)) : 0.0f;
      const float xA = __shfl_xor(sA, 32), xB = __shfl_xor(sB, 32);
      const float g = half == 0 ? sA : xB, u = half == 0 ? xA : sB;
      const bool live = half == 0 || two;
      const float hv = live ? g / (1.0f + expf(-g)) * u : 0.0f;
      float amax = fabsf(hv);
#pragma unroll
      for (int d = 1; d < 32; d <<= 1) amax = fmaxf(amax, __shfl_xor(amax, d));
      const int e = mx_exponent(amax, a.floor_rule != 0);
      const uint32_t code = to_e4m3(hv * exp2_neg(e));
      int jB = fj, cB = fc + 1;
      if (cB == ncols) {
        cB = 0;
        ++jB;
      }
      const int jj = half == 0 ? fj : jB, c2 = half == 0 ? fc : cB;
      if (live) {
        lds_st1(hb + c2 * m.hs + 32 * jj + hl, code);
        if (hl == 0) lds_st1(hb + 16 * m.hs + c2 * (a.IP / 32) + jj, static_cast<uint32_t>(e + 127));
        if (dump && a.dump_codes != nullptr) {
          const int pair = column_pair(m, lb, gi, c2);
          if (pair >= 0) {
            a.dump_codes[static_cast<int64_t>(pair) * a.I + 32 * jj + hl] = static_cast<uint8_t>(code);
            if (hl == 0) a.dump_scales[static_cast<int64_t>(pair) * (a.I / 32) + jj] = static_cast<uint8_t>(e + 127);
          }
        }
      }
      // advance past the entries just completed (one or two)
      fj = jB;
      fc = cB;
      if (two && ++fc == ncols) {
        fc = 0;
        ++fj;
      }
    }
    lds_settle();
  }
}

// The persistent routed-experts kernel (experts page, ExpertsKernel; runtime page,
// PersistentExperts.run): one workgroup per CU, co-resident (FC2 waits for hidden
// blocks that other workgroups' FC1 slices produce).  Waves 0-3 stream their items --
// FC1(A), FC1(B), FC2(A), FC2(B) -- through private LDS rings R items deep and touch
// global memory only through that DMA stream and the output stores, so no wait ever
// drains a ring.  Wave 4, the control wave, does every cross-workgroup step: it takes
// the streaming waves' FC1 sums of each block (LDS), files or finishes the block and
// publishes its hidden, then polls for the hidden of each FC2 chunk the workgroup
// needs and copies it into one of two LDS buffers.
// DEC: the decode form's prologue and LDS plan of x; TAG (decode form only): the FC1 ->
// FC2 exchange through tagged partial sums instead of finished hidden blocks.
template <int NT, int NS2, int R, bool DEC, bool TAG>
__global__ __launch_bounds__(kWG) void experts_kernel(ExpArgs a) {
  static_assert(DEC || !TAG, "the tagged exchange belongs to the decode form");
  using G = Geo<NT, R, NS2, DEC>;
  const int l = threadIdx.x & 63, w = wave_id(), grp = l >> 4;
  const LdsMap m = lds_map<NT, R, NS2, DEC>(static_cast<uint32_t>(a.g_cap), static_cast<uint32_t>(a.u_cap),
                                            static_cast<uint32_t>(a.IP), static_cast<uint32_t>(a.B),
                                            static_cast<uint32_t>(a.D));
  const uint32_t lb = lds_base();
  const uint32_t gen = a.calls[blockIdx.x];
  int n_groups, n_chunks;
  if constexpr (DEC) {
    n_groups = dec_route(a, m, kStream * R * G::SLOT);
    n_chunks = n_groups;  // one column tile per expert
  } else {
    n_groups = a.tbl.hdr[1];
    n_chunks = load_groups<NT>(a, m, n_groups, a.tbl.hdr[0]);
    fill_slices(a, m, n_groups, n_chunks);
    __syncthreads();
  }
  const uint32_t sy = lb + m.sync;
  agpr_form();

  if (w == kStream) {
    // ---------------------------------------------------------- control wave
    if constexpr (DEC)
      if (a.B * (a.D / 32) <= kPlanByControl) dec_plan_x(a, m, sy);
    v4f acc[4][NT];
    int q = 0;  // FC1 blocks of the workgroup taken so far
    for (int half = 0; half < 2; ++half) {
      const Slice S = slice_at(m, lb, half);
      if (S.hi <= S.lo) continue;
      for (int lbk = S.lo / a.NSP; lbk <= (S.hi - 1) / a.NSP; ++lbk, ++q) {
#pragma unroll
        for (int ww = 0; ww < kStream; ++ww) lds_wait<false>(sy + kSyncSub + 4 * ww, q + 1, a.err);
        // the streaming waves' sums, added in wave order
#pragma unroll
        for (int ww = 0; ww < (TAG ? 0 : kStream); ++ww)
#pragma unroll
          for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int n = 0; n < NT; ++n) {
              const uint4 v = lds_ld16(lb + m.red + ((((q & 1) * kStream + ww) * 4 + rt) * NT + n) * 1024 + l * 16);
              const v4f x = {__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w)};
              acc[rt][n] = ww == 0 ? x : acc[rt][n] + x;
            }
        if constexpr (TAG) {
          dec_publish(a, m, lb, n_groups, n_chunks, S, half, lbk, q, gen);
          if (l == 0) lds_st4(sy + kSyncAck, static_cast<uint32_t>(q + 1));
        } else {
          if (l == 0) lds_st4(sy + kSyncAck, static_cast<uint32_t>(q + 1));
          control_block<NT>(a, m, lb, n_groups, S, half, lbk, acc, gen);
        }
      }
    }
    int i = 0;  // FC2 chunks of the workgroup loaded so far
    for (int h = 2; h < 4; ++h) {
      SliceExtra sx;
      const Slice S2 = slice_at(m, lb, h, &sx);
      const int first = sx.span_first, cnt = sx.span_count;
      const int c_lo = h == 2 ? 0 : (n_chunks + 1) / 2;
      for (int c = first; c < first + cnt; ++c, ++i) {
        if (!TAG) wait_chunk(a, c, gen);
        if (i >= 2)  // buffer i&1 held chunk i-2: every wave must have moved past it
#pragma unroll
          for (int ww = 0; ww < kStream; ++ww) lds_wait<false>(sy + kSyncProg + 4 * ww, i - 1, a.err);
        if constexpr (TAG)
          dec_hidden(a, m, lb, n_groups, n_chunks, c, static_cast<uint32_t>(i & 1), S2.lo <= (c - c_lo) * a.U2, gen);
        else
          control_hidden<NT, NS2>(a, m, lb, n_groups, c, static_cast<uint32_t>(i & 1));
        if (l == 0) lds_st4(sy + kSyncReady + 4 * (i & 1), static_cast<uint32_t>(i));
      }
    }
    if (l == 0)
      for (int qq = blockIdx.x; qq < kMaxGrid; qq += gridDim.x) a.calls[qq] = gen + 1;
    return;
  }

  // ------------------------------------------------------------ streaming waves
  static_assert(NT == 1, "one 16-column tile per weight pass");
  v4f acc[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) acc[rt] = v4f{0.f, 0.f, 0.f, 0.f};
  // decode form: the control wave's plan of x is in LDS (it also frees the hand-over
  // area, its staging buffer); waited for before the first FC1 item or hand-over write
  bool x_ok = !DEC;
  auto wait_x = [&]() {
    if (!x_ok) {
      lds_wait<false>(sy + kSyncX, 1, a.err);
      x_ok = true;
    }
  };
  // FC1 blocks are handed over in the workgroup's order: half A's slice, then B's
  int sub_h = 0, sub_q = 0;
  Slice sub = slice_at(m, lb, 0);
  int sub_b = sub.lo / a.NSP, sub_last = sub.hi > sub.lo ? (sub.hi - 1) / a.NSP : sub_b - 1;
  // Hands the sums of the workgroup's FC1 blocks below global block `upto` to the control
  // wave, in the workgroup's block order (zeros for blocks without steps of this wave).
  auto hand_over = [&](int upto) {
    while (sub_h < 2) {
      if (sub_b <= sub_last) {
        if (sub.base + sub_b >= upto) break;
        wait_x();
        lds_wait<false>(sy + kSyncAck, sub_q - 1, a.err);  // slot sub_q&1 is free once block sub_q-2 is taken
        mfma_settle(acc[0], acc[1], acc[2], acc[3]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const v4f v = acc[rt];
          lds_st16(lb + m.red + (((sub_q & 1) * kStream + w) * 4 + rt) * 1024 + l * 16,
                   make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                              __float_as_uint(v[3])));
          acc[rt] = v4f{0.f, 0.f, 0.f, 0.f};
        }
        ++sub_q;
        if (l == 0) lds_st4(sy + kSyncSub + 4 * w, static_cast<uint32_t>(sub_q));
        ++sub_b;
      } else if (++sub_h < 2) {
        sub = slice_at(m, lb, 1);
        sub_b = sub.lo / a.NSP;
        sub_last = sub.hi > sub.lo ? (sub.hi - 1) / a.NSP : sub_b - 1;
      }
    }
  };

  // the plan (x codes and scales) as a buffer: padded columns and pads load zeros from
  // outside it (decode form: an empty buffer, for the pads)
  const __amdgpu_buffer_rsrc_t xrsrc = __builtin_amdgcn_make_buffer_rsrc(
      DEC ? static_cast<void*>(a.out) : const_cast<uint8_t*>(a.xcodes), static_cast<short>(0),
      DEC ? 0u : a.plan_bytes, 0x00020000);
  Cursor pc;  // issue cursor, R items ahead of consumption
  pc.h = -1;
  pc.s = pc.s_hi = 0;
  pc.b = pc.hi = 0;
  cursor_next<DEC>(a, m, lb, n_groups, n_chunks, pc);
  int n_real = 0;  // real items issued (they precede the dummies)
  auto issue_next = [&](int k) {
    issue_item<NS2, R, DEC>(a, m, lb, pc, k, xrsrc);
    if (pc.h < 4) {
      ++n_real;
      cursor_next<DEC>(a, m, lb, n_groups, n_chunks, pc);
    }
  };
  // FC2 state of the chunk in use: per lane, its output row (or -1) and its column's
  // places in the hidden buffer
  int cur_seq = -1, orow = -1;
  uint32_t hbl = 0, hbs = 0;
  const int col = l & 15;
  // decode form, FC1: the chunk whose x rows the lane's column addresses hold
  int x_chunk = -1;
  uint32_t pxl = 0, pxsl = 0;
#pragma unroll 1
  for (int k = 0; k < R; ++k) issue_next(k);  // R items in flight
  for (int kc = 0;; ++kc) {
    const bool real = kc < n_real;
    const int slot = kc % R;
    const uint32_t sa_ = lb + m.ring + (w * R + slot) * G::SLOT;
    // this item's and the next item's records (written at issue; no need to wait for data)
    uint4 meta = make_uint4(3u, 0u, 0u, 0u), nm = make_uint4(3u, 0u, 0u, 0u);
    if (real) {
      asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                   : "=&v"(meta), "=&v"(nm)
                   : "v"(lb + m.meta + (w * R + slot) * 16), "v"(lb + m.meta + (w * R + (kc + 1) % R) * 16)
                   : "memory");
      if (kc + 1 >= n_real) nm = make_uint4(3u, 0u, 0u, 0u);
    }
    const int type = __builtin_amdgcn_readfirstlane(static_cast<int>(meta.x));
    // hand over the sums of the workgroup's FC1 blocks before this item's block (all of
    // them for an FC2 item or at the end); normally already done after the previous item
    hand_over(type == 0 ? __builtin_amdgcn_readfirstlane(static_cast<int>(meta.y)) : 0x7fffffff);
    if (!real) break;
    wait_vm<G::VM>();  // item kc has landed (the R-1 younger items may still be in flight)
    if (type == 0) {
      Fc1Ops op;
      if constexpr (DEC) {
        const int xc = __builtin_amdgcn_readfirstlane(static_cast<int>(meta.z));
        const int xsp = __builtin_amdgcn_readfirstlane(static_cast<int>(meta.w));
        wait_x();
        if (xc != x_chunk) {
          x_chunk = xc;
          const GroupInfo xgi = group_of(m, lb, n_groups, xc);
          const int pair = column_pair(m, lb, xgi, xgi.cc * 16 + col);
          const int t = pair >= 0 ? pair / a.K : a.B;  // padded columns read the zero row
          pxl = lb + m.xq + t * m.xstr + 16 * grp;
          pxsl = lb + m.xs + t * m.xss;
        }
        fc1_read_dec(sa_ + l * 16, sa_ + l * 4, pxl + 256 * xsp, pxsl + 8 * xsp, op);
      } else {
        fc1_read(sa_ + l * 16, sa_ + l * 4, op);
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const v8i bop = fp8_operand(op.x[2 * st], op.x[2 * st + 1]);
        const int sb = static_cast<int>((op.xs[st] >> (8 * grp)) & 0xffu);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
          acc[rt] = mfma_fp4_fp8(fp4_operand(op.a[4 * st + rt]), bop, acc[rt],
                                 static_cast<int>((op.as[st] >> (8 * rt)) & 0xffu), sb);
      }
      // this wave's part of the block may be complete: the next item's record tells, so
      // the sums go to the control wave without waiting for the next item's data
      const int ntype = __builtin_amdgcn_readfirstlane(static_cast<int>(nm.x));
      hand_over(ntype == 0 ? __builtin_amdgcn_readfirstlane(static_cast<int>(nm.y)) : 0x7fffffff);
    } else if (type == 1) {
      constexpr int T2 = Fc2Tiles<NS2>::T2;
      const int seq = __builtin_amdgcn_readfirstlane(static_cast<int>(meta.w));
      if (seq != cur_seq) {
        if (l == 0) lds_st4(sy + kSyncProg + 4 * w, static_cast<uint32_t>(seq));
        lds_wait<true>(sy + kSyncReady + 4 * (seq & 1), seq, a.err);
        cur_seq = seq;
        const GroupInfo hgi = group_of(m, lb, n_groups, __builtin_amdgcn_readfirstlane(static_cast<int>(meta.y)));
        const int pair = column_pair(m, lb, hgi, hgi.cc * 16 + col);
        orow = pair >= 0 ? pair * a.D : -1;
        const uint32_t hb = lb + m.hid + static_cast<uint32_t>(seq & 1) * m.hid_bytes;
        hbl = hb + col * m.hs + 16 * grp;
        hbs = hb + 16 * m.hs + col * (a.IP / 32);
      }
      HidOps<NS2> hop;
      hid_read<NS2>(hbl, hbs, hop);
      Fc2Ops<NS2, T2> op;
      fc2_read<NS2, T2>(sa_ + l * 16, sa_ + l * 4, op);
      v8i bop[NS2];
      int sb[NS2];
#pragma unroll
      for (int s = 0; s < NS2; ++s) {
        // K-blocks beyond I (I not a multiple of 128) are zero
        const bool lo_ok = 4 * s + (grp >> 1) < a.HB, hi_ok = 4 * s + 2 + (grp >> 1) < a.HB;
        const bool sc_ok = 4 * s + grp < a.HB;
        const uint4 z = make_uint4(0, 0, 0, 0);
        bop[s] = fp8_operand(lo_ok ? hop.bl[s] : z, hi_ok ? hop.bh[s] : z);
        sb[s] = sc_ok ? static_cast<int>((hop.bs[s] >> (8 * grp)) & 0xffu) : 127;
      }
      v4f o[T2];
#pragma unroll
      for (int t = 0; t < T2; ++t) {
        o[t] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NS2; ++s)
          o[t] = mfma_fp4_fp8(fp4_operand(op.a[t * NS2 + s]), bop[s], o[t],
                              static_cast<int>((op.as[t] >> (8 * s)) & 0xffu), sb[s]);
      }
#pragma unroll
      for (int t = 0; t < T2; ++t) mfma_settle(o[t]);
      if (orow >= 0) {
        const int d0 = static_cast<int>(meta.z) * T2 * 16 + 4 * grp;
#pragma unroll
        for (int t = 0; t < T2; ++t) {
          const uint2 v = make_uint2(to_bf16_bits(o[t][0]) | (to_bf16_bits(o[t][1]) << 16),
                                     to_bf16_bits(o[t][2]) | (to_bf16_bits(o[t][3]) << 16));
          *reinterpret_cast<uint2*>(a.out + static_cast<int64_t>(orow) + d0 + 16 * t) = v;
        }
      }
    }
    issue_next(kc + R);  // into the slot just consumed
  }
  if (l == 0) lds_st4(sy + kSyncProg + 4 * w, 0x7fffffffu);  // done with every FC2 chunk
  // drain the dummy items before the workgroup ends
  wait_vm<0>();
}

// =================================================================== decode form, whole-K FC1 blocks
// moe_decode_run's default exchange.  A variant of the decode form in which no hidden
// block is ever split between workgroups:
//   * an FC1 item is one hidden block (distinct expert g, block j of 32 hidden values):
//     the 64 weight rows gate 32j..32j+31 and the matching up rows over the whole of K.
//     The workgroup's four streaming waves take every fourth 128-wide K step of it; the
//     control wave adds their four partial tiles in wave order, applies SwiGLU and the
//     MXFP8 requantization (experts page, ExpertsKernel.store_hidden) and publishes the
//     block with a call-tagged flag.  No FC1 partial sum leaves the workgroup.
//   * FC2 is dealt as 16-row output tiles, a contiguous run of them (in expert-major
//     order) per workgroup, so a workgroup's FC2 touches one or two experts; the tiles of
//     one expert wait for that expert's block flags only.
//   * FC1 items go round-robin too (item i to workgroup i mod grid); the workgroups with
//     one item fewer take proportionally more FC2 tiles, so every workgroup streams about
//     the same number of weight bytes (experts page, ExpertsKernel.partition, contiguous
//     near-equal shares of the weight stream).
// The weight stream of a streaming wave is one sequence of equal slots (an FC1 K step:
// four 1 KB row tiles and their scale words; or an FC2 tile: NS2 1 KB K steps and its
// scale words), R in flight through LDS DMA, so "the oldest slot has landed" is always
// the same vmcnt.

constexpr int kQSlot = 4096 + 256;  // slot bytes
constexpr int kQOps = 5;            // DMA instructions per slot (pads keep it fixed)
constexpr int kQGMax = 128;         // distinct experts per call
constexpr int kQXBlk = 4;           // 32-element x blocks per thread held in the prologue
constexpr int kQHB = 16;            // hidden scale slots per token column (HB <= 16)

constexpr int kQStream = 8;                  // streaming waves per workgroup
constexpr int kQFin = kQStream;             // the finisher wave: FC1 blocks' epilogues
constexpr int kQLoad = kQStream + 1;         // the loader wave: FC2's hidden, polled and copied
constexpr int kQPoll = 18;  // hidden pairs per loader lane, one-pass poll: 8 x (512 / 4 + 16) / 64
constexpr int kQWG = 64 * (kQStream + 2);

// LDS: sync words and the routing tables of the batch (byte offsets from the LDS base).
constexpr uint32_t kQProg = 0;      // [8] FC1 items whose partial tiles wave w has written
constexpr uint32_t kQProg2 = 32;    // [8] wave w is done with every FC2 hidden sequence < value
constexpr uint32_t kQCons = 64;     // FC1 items whose partial tiles the control wave has read
constexpr uint32_t kQReady = 68;    // FC2 hidden sequences loaded into the two hidden buffers
constexpr uint32_t kQXDone = 72;    // waves that have written their share of the x plan
constexpr uint32_t kQGCount = 76;   // distinct experts of the batch
constexpr uint32_t kQCall = 80;     // this call's number (tag of the published hidden)
constexpr uint32_t kQEmask = 128;   // [32] expert bitmask (E <= 1024)
constexpr uint32_t kQPre = 256;     // [32] popcount prefix of the bitmask words
constexpr uint32_t kQExp = 384;     // [kQGMax] expert id of group g (ascending)
constexpr uint32_t kQTok = 896;     // [kQGMax] token bitmask of group g
constexpr uint32_t kQRow = 1408;    // [kQGMax][8] u16: pair t*K+s of group g's column c
constexpr uint32_t kQTaken = 3456;  // [8] FC2 queue entries wave w's issue side has taken
constexpr uint32_t kQPosted = 3488; // FC2 queue entries the claimer has posted
constexpr uint32_t kQQueue = 3504;  // [kQRing] FC2 queue: first tile of a claimed grain, -1 = end
constexpr uint32_t kQTables = 3584;

// FC2 tail claims (experts page, ExpertsKernel: steal, claims, fc2_steal; runtime page,
// dynamic(batch): a static FC2 split leaves the slowest workgroup as the launch's tail).
// The last grains of each workgroup's FC2 run form its zone; a 64-bit counter per
// workgroup, {call, back claims, front claims}, hands each grain out once: the owner
// claims from the front, the workgroups before it in tile order from the back.
constexpr int kQGrain = kQStream;  // FC2 tiles of a grain: one per streaming wave
constexpr int kQZone = 4;          // most grains in a zone
constexpr int kQAhead = 4;         // grains the claimer posts ahead of the slowest issue side
constexpr int kQVictims = 2;       // workgroups after this one whose zones it may take from
constexpr int kQRing = 16;         // queue entries (more than kQAhead plus the ring depth)

// ---------------------------------------------------- next-layer weight prefetch
// Next-layer weight prefetch (runtime page, PersistentExperts.run's ahead table): rows of
// (address, bytes) of device memory the next launch reads.  Their bytes, cut into 1 KB
// pieces, are split evenly over the workgroups; one wave of each reads its share into 1 KB
// of LDS it no longer needs (bounds-checked buffer loads: a row's last piece reads
// nothing past its end).  What matters is the side effect: the bytes pass through, and
// stay in, the Infinity Cache, so that the next launch's first weight reads hit it.
constexpr int kPfRows = 64;    // rows of a table (kernel arguments hold it)
constexpr int kPfFlight = 32;  // pieces in flight per wave
struct PfRow {
  uint64_t addr;
  uint32_t bytes;
  uint32_t first;  // index of the row's first piece among all rows' pieces
};
struct PfTable {
  int rows, pieces;
  PfRow row[kPfRows];
};

__device__ __forceinline__ void pf_run(const PfTable& t, int c, int nwg, uint32_t dst) {
  const int64_t P = t.pieces;
  const int p0 = static_cast<int>(P * c / nwg), p1 = static_cast<int>(P * (c + 1) / nwg);
  const int l = threadIdx.x & 63;
  int r = 0, next = t.rows > 1 ? static_cast<int>(t.row[1].first) : p1;
  auto at = [&](int k) { return rsrc(reinterpret_cast<const void*>(t.row[k].addr), t.row[k].bytes); };
  __amdgpu_buffer_rsrc_t rs = at(0);
  int n = 0;
#pragma unroll 1
  for (int p = p0; p < p1; ++p) {
    if (p >= next) {
#pragma unroll 1
      while (r + 1 < t.rows && p >= static_cast<int>(t.row[r + 1].first)) ++r;
      next = r + 1 < t.rows ? static_cast<int>(t.row[r + 1].first) : p1;
      rs = at(r);
    }
    if (n >= kPfFlight) wait_vm<kPfFlight - 1>();
    sdma16(rs, static_cast<uint32_t>(p - static_cast<int>(t.row[r].first)) * 1024u + 16u * l, 0u, dst);
    ++n;
  }
  wait_vm<0>();
}

struct QArgs {
  const uint8_t* w13p;
  const uint8_t* s13p;
  const uint8_t* w2p;
  const uint8_t* s2p;
  const uint16_t* x;      // BF16 [B, D]
  const int32_t* ids;     // [B, K]
  uint16_t* out;          // BF16 [B*K, D]
  uint64_t* hq;           // [kQGMax][8][hq_words] the hidden as (data, call) pairs: per
                          // column I/4 code words, then HB scale words
  uint32_t* calls;        // [kMaxGrid] per-workgroup call counters
  uint64_t* claims;       // [kMaxGrid] per-workgroup FC2 claim counters {call, back, front}
  int32_t* err;           // status word (bit 0 id out of range, bit 1 repeated id, bit 2 a wait gave up)
  uint8_t* dump_codes;    // optional [B*K, I]
  uint8_t* dump_scales;   // optional [B*K, I/32]
  uint8_t* plan_dump;     // optional plan of x (moe_plan layout), written by workgroup 0
  int B, K, E, D, I, HB, NS1, IP, floor_rule, hq_words;
  int zone;               // most grains of a claimable FC2 zone (0: static FC2 runs)
  uint32_t o_red, o_hid, o_xq, o_xs, o_ring;  // LDS offsets
  uint32_t xstr, xsstr, hid_bytes;            // x code row stride, x scale row stride, one hidden buffer
  int cb;                 // token columns a group can have: min(B, 8); sizes the LDS areas below
  uint32_t red_wave;      // one wave's partial tiles: 4 tiles x cb columns x 16 rows x FP32
  PfTable pf;             // next-layer prefetch rows
};

// Four 16-byte LDS reads at four addresses, one wait.
__device__ __forceinline__ void lds_ld16x4v(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3, uint4& v0, uint4& v1,
                                            uint4& v2, uint4& v3) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3)
      : "memory");
}

// Two binary32 values to two BF16 (low half = a), round to nearest even
// (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(a))) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(b))) << 16);
}

__device__ __forceinline__ void lds_add4(uint32_t addr, uint32_t v) {
  asm volatile("ds_add_u32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : : "v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_st1_async(uint32_t addr, uint32_t v) {
  asm volatile("ds_write_b8 %0, %1" : : "v"(addr), "v"(v) : "memory");
}

// The workgroup's share of the work (the same on every lane; all workgroups agree).
struct QWork {
  int n1;      // FC1 items: i = c + k * grid, k < n1
  int m1;      // this wave's K steps per FC1 item (steps w, w + 8, ...; 0 for w >= NS1)
  int n2;      // FC2 tiles: the contiguous run first2 .. first2 + n2 - 1 (expert-major order)
  int first2;
  int TPE, nwg, c;
};

// FC2 tiles that stream as long as one FC1 item (34 / (NS2 + 1/4) per 1024 columns of D:
// an item's K steps against a tile's NS2 steps plus its scales).
__host__ __device__ inline int q_item_tiles(int D, int NS2) { return 34 * D / (NS2 * 1024 + 256); }

// Callable on the host too (moe_work_split evaluates it there for schedule checks).
__host__ __device__ inline QWork q_work(int G, int HB, int NS1, int D, int nwg, int c, int w, int item,
                                        int nst = kQStream) {
  QWork q;
  const int N1 = G * HB;
  q.nwg = nwg;
  q.c = c;
  q.TPE = D / 16;
  const int N2 = G * q.TPE;
  const int r1 = N1 % nwg;  // workgroups c < r1 hold one FC1 item more
  q.n1 = N1 / nwg + (c < r1 ? 1 : 0);
  q.m1 = w < NS1 ? (NS1 - w + nst - 1) / nst : 0;
  // FC2 tiles: contiguous runs in expert-major order.  When every workgroup has FC1
  // items and some have one more, those come last with `item` tiles fewer (an FC1 item
  // streams as long as that many FC2 tiles): they take the experts that finish last,
  // their own last items among them.  Otherwise (no FC1 item for some workgroups, or
  // the same count for all) the runs are equal: no FC2 tile can start before the last
  // round's hidden is there.
  int first, n2;
  if (N1 >= nwg && r1 > 0) {
    const int M0 = nwg - r1;  // workgroups with the fewer items: the first runs
    int cn = (N2 + r1 * item + nwg - 1) / nwg, ce = cn - item;
    if (ce <= 0) {
      cn = (N2 + M0 - 1) / M0;
      ce = 0;
    }
    // the workgroups with one item more take the last r1 * ce tiles, the others the
    // rest (M0 * cn covers it)
    const int e0 = N2 - r1 * ce > 0 ? N2 - r1 * ce : 0;
    if (c >= r1) {
      first = (c - r1) * cn < e0 ? (c - r1) * cn : e0;
      n2 = e0 - first < cn ? e0 - first : cn;
    } else {
      const int a0 = N2 - (r1 - c) * ce, a1 = N2 - (r1 - c - 1) * ce;
      first = a0 > 0 ? a0 : 0;
      n2 = (a1 > 0 ? a1 : 0) - first;
    }
  } else {
    const int cap = (N2 + nwg - 1) / nwg;
    first = c * cap;
    n2 = cap;
  }
  q.first2 = first < N2 ? first : N2;
  n2 = N2 - q.first2 < n2 ? N2 - q.first2 : n2;
  q.n2 = n2 < 0 ? 0 : n2;
  return q;
}

// The claimable zone of a workgroup's FC2 run: its last Z grains, Z at most `zone` and
// at most half the run.  Only runs of at least 16 R tiles have one, so that every
// streaming wave's static head holds R tiles or more: a wave's issue side, R slots ahead,
// then reaches the claimed grains only once its FC1 slots are consumed (the claimer is
// the finisher wave, busy with FC1 until then).  Returns Z; zb = the zone's first tile.
__host__ __device__ inline int q_zone(const QWork& q, int zone, int R, int& zb) {
  int Z = q.n2 >= 16 * R ? q.n2 / (2 * kQGrain) : 0;
  Z = Z < zone ? Z : zone;
  zb = q.first2 + q.n2 - Z * kQGrain;
  return Z;
}

// A streaming wave's walk over its FC2 tiles: the head of the run (tiles w, w + 8, ...
// below the zone), then tile w of each grain the claimer queues, until the end entry.
// The issue side waits for each entry to be posted and reports it taken; the consume
// side, R slots behind, reads entries already there.
struct QTiles {
  int t;        // next head tile
  int zb;       // first tile of the zone
  int q;        // next queue entry
  int s;        // -2 once the end entry is read
  int g, rt2;   // group and row tile of the next head tile (stepped without divisions)
};

__device__ __forceinline__ void q_tiles_init(QTiles& c, const QWork& q, int zb, int w) {
  c.t = q.first2 + w;
  c.zb = zb;
  c.q = 0;
  c.s = -1;
  c.g = c.t / q.TPE;
  c.rt2 = c.t - c.g * q.TPE;
}

// The next tile: true with its group g and row tile rt2, false at the end (without
// claims, the end of the head).
template <bool ISSUE, bool CLAIMS>
__device__ __forceinline__ bool q_next_tile(uint32_t lb, int w, int TPE, QTiles& c, int32_t* err, int& g, int& rt2) {
  if (c.t < c.zb) {
    g = c.g;
    rt2 = c.rt2;
    c.t += kQStream;
    c.rt2 += kQStream;
#pragma unroll 1
    while (c.rt2 >= TPE) {
      c.rt2 -= TPE;
      ++c.g;
    }
    return true;
  }
  if (!CLAIMS || c.s == -2) return false;
  if (ISSUE) lds_wait<false>(lb + kQPosted, c.q + 1, err);
  const int s = static_cast<int>(lds_uni(lb + kQQueue + 4 * static_cast<uint32_t>(c.q % kQRing)));
  ++c.q;
  if (ISSUE && (threadIdx.x & 63) == 0) lds_st4(lb + kQTaken + 4 * w, static_cast<uint32_t>(c.q));
  if (s < 0) {
    c.s = -2;
    return false;
  }
  g = (s + w) / TPE;  // a claimed grain (claims only)
  rt2 = s + w - g * TPE;
  return true;
}

// One claim on a zone counter (lane 0's device-scope add; the old value to every lane).
__device__ __forceinline__ uint64_t q_claim(uint64_t* ctr, uint64_t inc) {
  uint64_t v = 0;
  if ((threadIdx.x & 63) == 0) v = __hip_atomic_fetch_add(ctr, inc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// The issue side of a streaming wave's slot sequence: its FC1 K steps (item by item),
// then its FC2 tiles (QTiles), then dummies (out-of-range loads that write zeros and
// read no memory, so the vmcnt of a slot stays fixed).
struct QIssue {
  int k;          // slots issued
  int item, si;   // next FC1 step: item of the workgroup, step index (s = w + 8 si)
  int64_t step;   // its packed step index ((e * HB + j) * NS1 + s)
  QTiles tl;      // FC2 tiles
  int g2, e2;     // group of the last FC2 tile issued and its expert
};

template <int NS2, int R, bool CLAIMS>
__device__ __forceinline__ void q_issue(const QArgs& a, const QWork& q, uint32_t lb, int w, int n1el,
                                        QIssue& is, __amdgpu_buffer_rsrc_t none) {
  const int l = threadIdx.x & 63;
  const uint32_t so = a.o_ring + static_cast<uint32_t>((w * R + is.k % R) * kQSlot);
  if (is.k < n1el) {
    if (is.si == 0) {
      const int i = q.c + is.item * q.nwg, g = i / a.HB, j = i - g * a.HB;
      const int e = lds_uni(lb + kQExp + 4 * g);
      is.step = (static_cast<int64_t>(e) * a.HB + j) * a.NS1 + w;
    }
    const uint8_t* wb = a.w13p + is.step * 4096 + l * 16;
#pragma unroll
    for (int t = 0; t < 4; ++t) dma16(wb + t * 1024, so + t * 1024);
    dma4(a.s13p + is.step * 256 + l * 4, so + 4096);
    is.step += kQStream;
    if (++is.si == q.m1) {
      is.si = 0;
      ++is.item;
    }
  } else if (int g = 0, rt2 = 0; q_next_tile<true, CLAIMS>(lb, w, q.TPE, is.tl, a.err, g, rt2)) {
    if (g != is.g2) {
      is.g2 = g;
      is.e2 = lds_uni(lb + kQExp + 4 * g);
    }
    const int64_t tile = static_cast<int64_t>(is.e2) * q.TPE + rt2;
    const uint8_t* wb = a.w2p + tile * NS2 * 1024 + l * 16;
#pragma unroll
    for (int s = 0; s < NS2; ++s) dma16(wb + s * 1024, so + s * 1024);
#pragma unroll
    for (int s = NS2; s < 4; ++s) bdma16(none, kOutside, so + s * 1024);
    dma4(a.s2p + tile * 256 + l * 4, so + 4096);
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) bdma16(none, kOutside, so + s * 1024);
    bdma4(none, kOutside, so + 4096);
  }
  ++is.k;
}

template <int NS2, int R, bool WIDE, bool CLAIMS>
__global__ __launch_bounds__(kQWG) void decode_whole_kernel(QArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  agpr_form();
  const int tid = threadIdx.x, l = tid & 63, w = wave_id();
  const int grp = l >> 4, col = l & 15;
  const uint32_t lb = lds_base();
  const int nwg = gridDim.x, c = blockIdx.x;
  const int D = a.D, HB = a.HB, NS1 = a.NS1, K = a.K, IP = a.IP;
  const int nkb = D / 32, nxb = a.B * nkb, nroutes = a.B * K;
  uint32_t* sw = reinterpret_cast<uint32_t*>(smem);

  // ---- prologue: ids, raw x rows and the call number in flight together
  if (tid < 21) sw[tid] = 0u;  // sync words and the call number
  if (CLAIMS && tid < 9) sw[kQTaken / 4 + tid] = 0u;  // the FC2 queue's taken and posted counts
  // the two hidden buffers start as zero codes with unit scales: the K-blocks past I (I
  // not a multiple of 128) then multiply zero-padded weights by zero, and the token
  // columns past a group's count hold finite values (their outputs are never stored)
  for (int v = tid; v < static_cast<int>(a.hid_bytes / 2); v += kQWG) {
    const uint32_t off = 4u * static_cast<uint32_t>(v), in_buf = off % a.hid_bytes;
    sw[(a.o_hid + off) / 4] = in_buf < static_cast<uint32_t>(a.cb * IP) ? 0u : 0x7f7f7f7fu;
  }
  if (tid < 32) sw[kQEmask / 4 + tid] = 0u;
  if (tid < kQGMax) sw[kQTok / 4 + tid] = 0u;
  int myid = -1;
  if (tid < nroutes) myid = a.ids[tid];
  uint32_t xw[kQXBlk][16];
#pragma unroll
  for (int i = 0; i < kQXBlk; ++i) {
    const int blk = tid + i * kQWG;
    if (blk < nxb) {
      const uint4* src = reinterpret_cast<const uint4*>(a.x + static_cast<int64_t>(blk) * 32);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint4 u = src[v];
        xw[i][4 * v] = u.x; xw[i][4 * v + 1] = u.y; xw[i][4 * v + 2] = u.z; xw[i][4 * v + 3] = u.w;
      }
    }
  }
  if (w == kQFin && l == 0) {
    const uint32_t call = ld_dev_u32(a.calls + c) + 1u;  // stored back at the end
    sw[kQCall / 4] = call;
    // re-arm this workgroup's claim counter for the call, {call, 0 back, 0 front}, early:
    // claims by others that reach it first see the old call's tag and take nothing
    if (CLAIMS) st_dev_u64(a.claims + c, static_cast<uint64_t>(call) << 32);
  }
  __syncthreads();

  // ---- routing (experts page, the capacity <= 8 path: one unit per distinct expert,
  // experts ascending, tokens in token order)
  const bool valid = myid >= 0 && myid < a.E;
  if (tid < nroutes) {
    if (!valid) __hip_atomic_fetch_or(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else atomicOr(sw + kQEmask / 4 + (myid >> 5), 1u << (myid & 31));
  }
  __syncthreads();
  if (tid < 32) {
    const int pc = __popc(sw[kQEmask / 4 + tid]);
    int inc = pc;
#pragma unroll
    for (int d = 1; d < 32; d <<= 1) {
      const int o = __shfl_up(inc, d);
      if (l >= d) inc += o;
    }
    sw[kQPre / 4 + tid] = static_cast<uint32_t>(inc - pc);
    if (tid == 31) sw[kQGCount / 4] = static_cast<uint32_t>(inc);
  }
  __syncthreads();
  int g_mine = -1;
  if (tid < nroutes && valid) {
    const uint32_t word = sw[kQEmask / 4 + (myid >> 5)];
    g_mine = static_cast<int>(sw[kQPre / 4 + (myid >> 5)]) + __popc(word & ((1u << (myid & 31)) - 1u));
    const int t = tid / K;
    const uint32_t old = atomicOr(sw + kQTok / 4 + g_mine, 1u << t);
    if (old & (1u << t)) __hip_atomic_fetch_or(a.err, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sw[kQExp / 4 + g_mine] = static_cast<uint32_t>(myid);
  }
  __syncthreads();
  if (g_mine >= 0) {
    const int t = tid / K;
    const int cc = __popc(sw[kQTok / 4 + g_mine] & ((1u << t) - 1u));
    reinterpret_cast<uint16_t*>(smem + kQRow)[g_mine * 8 + cc] = static_cast<uint16_t>(tid);
  }
  const int G = __builtin_amdgcn_readfirstlane(static_cast<int>(sw[kQGCount / 4]));
  __syncthreads();

  const int item_tiles = q_item_tiles(D, NS2);
  const QWork q = q_work(G, HB, NS1, D, nwg, c, w < kQStream ? w : 0, item_tiles);
  const __amdgpu_buffer_rsrc_t none =
      __builtin_amdgcn_make_buffer_rsrc(static_cast<void*>(a.out), static_cast<short>(0), 0u, 0x00020000);
  const int nw1 = NS1 < kQStream ? NS1 : kQStream;  // waves that take FC1 steps
  int zb = q.first2 + q.n2;
  const int Z = CLAIMS ? q_zone(q, a.zone, R, zb) : 0;  // this workgroup's claimable FC2 grains
  // without a zone the queue holds only its end entry, posted before anything can wait
  // for it
  if (CLAIMS && Z == 0 && w == kQFin && l == 0) {
    lds_st4(lb + kQQueue, 0xffffffffu);
    lds_st4(lb + kQPosted, 1u);
  }

  // ---- streaming waves start their weight streams; the x plan does not gate them
  const int n1el = w < kQStream ? q.n1 * q.m1 : 0;
  QIssue is;
  is.k = 0;
  is.item = is.si = 0;
  is.step = 0;
  q_tiles_init(is.tl, q, zb, w);
  is.g2 = -1;
  is.e2 = 0;
  if (w < kQStream) {
#pragma unroll 1
    for (int k = 0; k < R; ++k) q_issue<NS2, R, CLAIMS>(a, q, lb, w, n1el, is, none);
  }

  // ---- the MXFP8 plan of x (experts page, plan_chunk / mx_block), all waves, into LDS
#pragma unroll
  for (int i = 0; i < kQXBlk; ++i) {
    const int blk = tid + i * kQWG;
    if (blk < nxb) {
      uint32_t cw[8];
      const int e = mx_block32_hw(xw[i], cw);
      const int t = blk / nkb, kb = blk - t * nkb;
      const uint32_t dst = lb + a.o_xq + t * a.xstr + 32 * kb;
      lds_st16_async(dst, make_uint4(cw[0], cw[1], cw[2], cw[3]));
      lds_st16_async(dst + 16, make_uint4(cw[4], cw[5], cw[6], cw[7]));
      lds_st1_async(lb + a.o_xs + t * a.xsstr + kb, static_cast<uint32_t>(e + 127));
      if (a.plan_dump != nullptr && c == 0) {
        uint4* pd = reinterpret_cast<uint4*>(a.plan_dump + static_cast<int64_t>(blk) * 32);
        pd[0] = make_uint4(cw[0], cw[1], cw[2], cw[3]);
        pd[1] = make_uint4(cw[4], cw[5], cw[6], cw[7]);
        a.plan_dump[static_cast<int64_t>(nxb) * 32 + blk] = static_cast<uint8_t>(e + 127);
      }
    }
  }
  lds_settle_all();
  if (l == 0) lds_add4(lb + kQXDone, 1u);

  const int g0 = q.first2 / q.TPE;  // expert of the workgroup's first FC2 tile (sequence 0)

  if (w < kQStream) {
    // =============================================================== streaming wave
    int k = 0;
    if (n1el > 0) lds_wait<false>(lb + kQXDone, kQStream + 2, a.err);
    // ---- FC1: this wave's K steps of each of the workgroup's hidden blocks
#pragma unroll 1
    for (int item = 0; item < q.n1 && q.m1 > 0; ++item) {
      uint32_t px, pxs;
      bool xlive;
      {
        const int i = q.c + item * q.nwg, g = i / HB;
        const int ng = __popc(static_cast<int>(lds_ld4(lb + kQTok + 4 * g)));
        xlive = col < ng;
        int t = 0;
        if (xlive) t = static_cast<int>(lds_ld2(lb + kQRow + 2 * (g * 8 + col))) / K;
        px = lb + a.o_xq + t * a.xstr + 16 * grp + 128 * w;
        pxs = lb + a.o_xs + t * a.xsstr + 4 * w;
      }
      v4f acc[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) acc[rt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
      for (int si = 0; si < q.m1; ++si, ++k) {
        wait_vm<(R - 1) * kQOps>();  // slot k has landed (the R - 1 younger ones may be in flight)
        const uint32_t sa = lb + a.o_ring + static_cast<uint32_t>((w * R + k % R) * kQSlot);
        uint4 a0, a1, a2, a3, xl, xh;
        uint32_t as, xs;
        asm volatile(
            "ds_read_b128 %0, %8 offset:0\n\t"
            "ds_read_b128 %1, %8 offset:1024\n\t"
            "ds_read_b128 %2, %8 offset:2048\n\t"
            "ds_read_b128 %3, %8 offset:3072\n\t"
            "ds_read_b32 %4, %9 offset:4096\n\t"
            "ds_read_b128 %5, %10 offset:0\n\t"
            "ds_read_b128 %6, %10 offset:64\n\t"
            "ds_read_b32 %7, %11 offset:0\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3), "=&v"(as), "=&v"(xl), "=&v"(xh), "=&v"(xs)
            : "v"(sa + l * 16), "v"(sa + l * 4), "v"(px + 1024 * si), "v"(pxs + 32 * si)
            : "memory");
        // columns past the group's tokens read token 0's row: their sums are never used
        const v8i bop = fp8_operand(xl, xh);
        const int sb = static_cast<int>((xs >> (8 * grp)) & 0xffu);
        acc[0] = mfma_fp4_fp8(fp4_operand(a0), bop, acc[0], static_cast<int>(as & 0xffu), sb);
        acc[1] = mfma_fp4_fp8(fp4_operand(a1), bop, acc[1], static_cast<int>((as >> 8) & 0xffu), sb);
        acc[2] = mfma_fp4_fp8(fp4_operand(a2), bop, acc[2], static_cast<int>((as >> 16) & 0xffu), sb);
        acc[3] = mfma_fp4_fp8(fp4_operand(a3), bop, acc[3], static_cast<int>(as >> 24), sb);
        q_issue<NS2, R, CLAIMS>(a, q, lb, w, n1el, is, none);  // into the slot just consumed
      }
      // the wave's part of the block is done: hand its partial tiles (the block's token
      // columns) to the finisher once it has taken the last ones
      mfma_settle(acc[0], acc[1], acc[2], acc[3]);
      lds_wait<false>(lb + kQCons, item, a.err);
      if (xlive) {  // the live token columns (col < ng <= cb)
        const uint32_t rd = lb + a.o_red + w * a.red_wave + static_cast<uint32_t>((grp * a.cb + col) * 16);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
          lds_st16_async(rd + rt * 64 * a.cb, make_uint4(__float_as_uint(acc[rt][0]), __float_as_uint(acc[rt][1]),
                                                   __float_as_uint(acc[rt][2]), __float_as_uint(acc[rt][3])));
      }
      lds_settle_all();
      if (l == 0) lds_st4(lb + kQProg + 4 * w, static_cast<uint32_t>(item + 1));
    }

    // ---- FC2: this wave's tiles of the workgroup's run (w, w + 8, ... of its head, then
    // tile w of each claimed grain)
    int cur_seq = -1, orow = -1;
    uint32_t hbl = 0, hbs = 0;
    QTiles ct;
    q_tiles_init(ct, q, zb, w);
#pragma unroll 1
    for (;; ++k) {
      int g = 0, rt2 = 0;
      if (!q_next_tile<false, CLAIMS>(lb, w, q.TPE, ct, a.err, g, rt2)) break;
      wait_vm<(R - 1) * kQOps>();
      const uint32_t sa = lb + a.o_ring + static_cast<uint32_t>((w * R + k % R) * kQSlot);
      const int seq = g - g0;
      if (seq != cur_seq) {
        cur_seq = seq;
        if (l == 0) lds_st4(lb + kQProg2 + 4 * w, static_cast<uint32_t>(cur_seq));
        const int tok = static_cast<int>(lds_ld4(lb + kQTok + 4 * g));
        orow = -1;
        if (col < __popc(tok)) orow = static_cast<int>(lds_ld2(lb + kQRow + 2 * (g * 8 + col))) * D;
        const uint32_t hb = lb + a.o_hid + static_cast<uint32_t>(cur_seq & 1) * a.hid_bytes;
        const int hcol = orow >= 0 ? col : 0;  // other lanes read column 0 and use zeros
        hbl = hb + hcol * IP + 16 * grp;
        hbs = hb + a.cb * IP + hcol * kQHB;
        lds_wait<false>(lb + kQReady, cur_seq + 1, a.err);
      }
      uint4 wa0, wa1, wa2, wa3;
      uint32_t was;
      asm volatile(
          "ds_read_b128 %0, %5 offset:0\n\t"
          "ds_read_b128 %1, %5 offset:1024\n\t"
          "ds_read_b128 %2, %5 offset:2048\n\t"
          "ds_read_b128 %3, %5 offset:3072\n\t"
          "ds_read_b32 %4, %6 offset:4096\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(wa0), "=&v"(wa1), "=&v"(wa2), "=&v"(wa3), "=&v"(was)
          : "v"(sa + l * 16), "v"(sa + l * 4)
          : "memory");
      const uint4 wa[4] = {wa0, wa1, wa2, wa3};
      HidOps<NS2> hop;
      hid_read<NS2>(hbl, hbs, hop);
      const bool live = orow >= 0;
      v4f o = v4f{0.f, 0.f, 0.f, 0.f};
      // K-blocks past I hold zero codes (weights and hidden); columns past the group's
      // tokens read column 0 and are not stored
#pragma unroll
      for (int s = 0; s < NS2; ++s)
        o = mfma_fp4_fp8(fp4_operand(wa[s]), fp8_operand(hop.bl[s], hop.bh[s]), o,
                         static_cast<int>((was >> (8 * s)) & 0xffu), static_cast<int>((hop.bs[s] >> (8 * grp)) & 0xffu));
      mfma_settle(o);
      if (live) {
        // FP32 -> BF16 round to nearest even with gfx950's packed conversion
        const uint2 v = make_uint2(bf16_pair(o[0], o[1]), bf16_pair(o[2], o[3]));
        *reinterpret_cast<uint2*>(a.out + static_cast<int64_t>(orow) + 16 * rt2 + 4 * grp) = v;
      }
      q_issue<NS2, R, CLAIMS>(a, q, lb, w, n1el, is, none);
    }
    if (l == 0) lds_st4(lb + kQProg2 + 4 * w, 0x7fffffffu);
    wait_vm<0>();  // the dummy slots land before the workgroup ends
    return;
  }

  const uint32_t call = static_cast<uint32_t>(lds_uni(lb + kQCall));
  if (w == kQFin) {
    // =============================================================== finisher wave
    // the control waves issue ahead of the streaming waves on their SIMDs: the finisher's
    // SwiGLU and requantization, and the loader's polls, are on the step's critical path
    __builtin_amdgcn_s_setprio(2);
    // FC1: finish the workgroup's hidden blocks in order
#pragma unroll 1
  for (int k = 0; k < q.n1; ++k) {
    const int i = q.c + k * q.nwg, g = i / HB, j = i - g * HB;
    v4f tot[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) tot[rt] = v4f{0.f, 0.f, 0.f, 0.f};
    const int tok = static_cast<int>(lds_ld4(lb + kQTok + 4 * g));
    const bool live = col < __popc(tok);  // the block's token columns
    const uint32_t rd = lb + a.o_red + static_cast<uint32_t>((grp * a.cb + col) * 16);
    // each wave's partial tiles are added (in wave order) as soon as that wave posts them
#pragma unroll 1
    for (int ww = 0; ww < nw1; ++ww) {
      lds_wait<false>(lb + kQProg + 4 * ww, k + 1, a.err);
      if (live) {
        uint4 p0, p1, p2, p3;
        const uint32_t rw = rd + ww * a.red_wave, ts = 64u * a.cb;
        lds_ld16x4v(rw, rw + ts, rw + 2 * ts, rw + 3 * ts, p0, p1, p2, p3);
        const uint4 p[4] = {p0, p1, p2, p3};
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          tot[rt][0] += __uint_as_float(p[rt].x);
          tot[rt][1] += __uint_as_float(p[rt].y);
          tot[rt][2] += __uint_as_float(p[rt].z);
          tot[rt][3] += __uint_as_float(p[rt].w);
        }
      }
    }
    if (l == 0) lds_st4(lb + kQCons, static_cast<uint32_t>(k + 1));
    // SwiGLU and MXFP8 of the block (experts page, store_hidden): lane (col, grp) holds
    // hidden values 32j + 4grp + r (tile 0) and 32j + 16 + 4grp + r (tile 1) of column col
    float h[2][4];
    float amax = 0.0f;
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float gv = tot[half][r], uv = tot[2 + half][r];
        // SwiGLU with the hardware exponential and reciprocal (a few ulp in FP32; the
        // hidden is then rounded to 3 mantissa bits)
        h[half][r] = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
        amax = fmaxf(amax, fabsf(h[half][r]));
      }
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    const int e = mx_exponent(amax, a.floor_rule != 0);
    const float sc = exp2_neg(e);
    uint32_t word[2];
    auto clampf = [](float v) { return fminf(fmaxf(v, -448.0f), 448.0f); };  // the floor rule saturates
#pragma unroll
    for (int half = 0; half < 2; ++half)
      word[half] = cvt4_e4m3(clampf(h[half][0] * sc), clampf(h[half][1] * sc), clampf(h[half][2] * sc),
                             clampf(h[half][3] * sc));
    if (live) {
      // (data, call) pairs: one 8-byte device-coherent store carries a word and its tag,
      // so no flag and no wait for the stores are needed
      uint64_t* hq = a.hq + (static_cast<int64_t>(g) * 8 + col) * a.hq_words;
      const uint64_t tag = static_cast<uint64_t>(call) << 32;
      st_dev_u64(hq + 8 * j + grp, tag | word[0]);
      st_dev_u64(hq + 8 * j + 4 + grp, tag | word[1]);
      if (grp == 0) st_dev_u64(hq + a.I / 4 + j, tag | static_cast<uint32_t>(e + 127));
      if (a.dump_codes != nullptr) {
        const int pair = static_cast<int>(lds_ld2(lb + kQRow + 2 * (g * 8 + col)));
        uint8_t* dc = a.dump_codes + static_cast<int64_t>(pair) * a.I + 32 * j + 4 * grp;
        *reinterpret_cast<uint32_t*>(dc) = word[0];
        *reinterpret_cast<uint32_t*>(dc + 16) = word[1];
        if (grp == 0) a.dump_scales[static_cast<int64_t>(pair) * HB + j] = static_cast<uint8_t>(e + 127);
      }
    }
  }

    if (CLAIMS && Z > 0) {
      // FC2 tail claims: queue this workgroup's zone grains from the front, then grains
      // of the zones of the next workgroups from the back where all their tiles belong to
      // this workgroup's last expert (whose hidden its last buffer keeps), then the end.
      // Each claim waits until every streaming wave has taken all but kQAhead of the
      // posted grains, so grains stay unclaimed, and free for others, until needed.  A
      // grain is computed by whoever claims it exactly as its owner would.
      int posted = 0;
      auto pace = [&]() {
        if (posted >= kQAhead) {
#pragma unroll 1
          for (int ww = 0; ww < kQStream; ++ww) lds_wait<false>(lb + kQTaken + 4 * ww, posted - kQAhead + 1, a.err);
        }
      };
      auto post = [&](int first) {
        if (l == 0) {
          lds_st4(lb + kQQueue + 4 * static_cast<uint32_t>(posted % kQRing), static_cast<uint32_t>(first));
          lds_st4(lb + kQPosted, static_cast<uint32_t>(posted + 1));
        }
        ++posted;
      };
#pragma unroll 1
      for (;;) {
        pace();
        const uint64_t v = q_claim(a.claims + c, 1u);
        const int f = static_cast<int>(v & 0xffffu), r = static_cast<int>((v >> 16) & 0xffffu);
        if (static_cast<uint32_t>(v >> 32) != call || f + r >= Z) break;
        post(zb + f * kQGrain);
      }
      const int glast = (q.first2 + q.n2 - 1) / q.TPE;
#pragma unroll 1
      for (int vc = c + 1; vc <= c + kQVictims && vc < nwg; ++vc) {
        const QWork qv = q_work(G, HB, NS1, D, nwg, vc, 0, item_tiles);
        int zbv = 0;
        const int Zv = q_zone(qv, a.zone, R, zbv);
        if (Zv == 0 || zbv / q.TPE != glast || (qv.first2 + qv.n2 - 1) / q.TPE != glast) continue;
#pragma unroll 1
        for (;;) {
          pace();
          const uint64_t v = q_claim(a.claims + vc, 1u << 16);
          const int f = static_cast<int>(v & 0xffffu), r = static_cast<int>((v >> 16) & 0xffffu);
          if (static_cast<uint32_t>(v >> 32) != call || f + r >= Zv) break;
          post(zbv + (Zv - 1 - r) * kQGrain);
        }
      }
      post(-1);
    }
    // the call counters for the next call (which starts after this kernel has ended, so
    // nothing waits on the stores): every counter c, c + grid, c + 2 grid, ... below
    // kMaxGrid, so all of them stay equal whatever grid the next call uses
#pragma unroll 1
    for (int m = c + l * nwg; m < kMaxGrid; m += 64 * nwg) st_dev_u32(a.calls + m, call);
    // next-layer weights: the workgroup's share, into the partial-sum area (free now)
    if (a.pf.pieces > 0) pf_run(a.pf, c, nwg, a.o_red);
    return;
  }
  // ================================================================= loader wave
  __builtin_amdgcn_s_setprio(2);  // as the finisher
  static_assert(kQLoad == kQStream + 1 && kQWG == 64 * (kQLoad + 1), "the loader is the last wave");
  // FC2: for each expert of the workgroup's run, in order, wait for its hidden (polling
  // from the start of the call) and copy it into one of the two LDS hidden buffers.  These
  // polls give up after kPollLimit rounds without reading the status word: a status read
  // in these loops lengthened the decode step by about a microsecond.
  const int nseq = q.n2 > 0 ? (q.first2 + q.n2 - 1) / q.TPE - g0 + 1 : 0;
#pragma unroll 1
  for (int seq = 0; seq < nseq; ++seq) {
    const int g = g0 + seq;
    if (seq >= 2) {
#pragma unroll 1
      for (int ww = 0; ww < kQStream; ++ww) lds_wait<false>(lb + kQProg2 + 4 * ww, seq - 1, a.err);
    }
    // load the expert's (data, call) pairs until every one carries this call's tag
    const int ng = __popc(static_cast<int>(lds_ld4(lb + kQTok + 4 * g)));
    const uint32_t hb = lb + a.o_hid + static_cast<uint32_t>(seq & 1) * a.hid_bytes;
    const uint64_t* src = a.hq + static_cast<int64_t>(g) * 8 * a.hq_words;
    const int per_col = a.I / 4 + HB;  // pairs a column holds: code words, then scales
    const int n = ng * per_col;
    if constexpr (WIDE) {
      // lane l holds pairs l, l + 64, ...: all of them are polled in each round, so an
      // expert of many tokens costs one round trip, not one per 512 pairs (a separate
      // variant: the longer loop slows the small batches, whose experts fit one round); the pair's
      // column and word advance by 64 = q64 columns + r64 words per step
      const int nu = (n + 63) >> 6;  // steps that hold pairs (uniform)
      const int q64 = 64 / per_col, r64 = 64 - q64 * per_col;
      const int c0 = l / per_col, w0 = l - c0 * per_col;
      uint64_t v[kQPoll];
  #pragma unroll 1
      for (uint32_t spins = 0;; ++spins) {
        int cc = c0, r = w0;
  #pragma unroll
        for (int u = 0; u < kQPoll; ++u) {
          v[u] = 0ull;
          if (u < nu) {  // uniform: the steps past the expert's pairs are skipped
            if (u * 64 + l < n) v[u] = ld_dev_u64(src + static_cast<int64_t>(cc) * a.hq_words + r);
            r += r64;
            cc += q64;
            const bool wrap = r >= per_col;
            r = wrap ? r - per_col : r;
            cc = wrap ? cc + 1 : cc;
          }
        }
        bool ok = true;
  #pragma unroll
        for (int u = 0; u < kQPoll; ++u) ok = ok && (u * 64 + l >= n || static_cast<uint32_t>(v[u] >> 32) == call);
        if (__all(ok)) break;
        if (spins == kPollLimit) {
          if (l == 0) __hip_atomic_fetch_or(a.err, 4, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      {
        int cc = c0, r = w0;
  #pragma unroll
        for (int u = 0; u < kQPoll; ++u) {
          if (u < nu) {
            if (u * 64 + l < n) {
              const uint32_t d = static_cast<uint32_t>(v[u]);
              if (r < a.I / 4) lds_st4_nw(hb + cc * IP + 4 * r, d);
              else lds_st1(hb + a.cb * IP + cc * kQHB + (r - a.I / 4), d);
            }
            r += r64;
            cc += q64;
            const bool wrap = r >= per_col;
            r = wrap ? r - per_col : r;
            cc = wrap ? cc + 1 : cc;
          }
        }
      }
    } else {
  #pragma unroll 1
      for (int base = 0; base < n; base += 8 * 64) {
        uint64_t v[8];
  #pragma unroll 1
        for (uint32_t spins = 0;; ++spins) {
          bool ok = true;
  #pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int idx = base + u * 64 + l;
            const int cc = idx / per_col, r = idx - cc * per_col;
            v[u] = idx < n ? ld_dev_u64(src + static_cast<int64_t>(cc) * a.hq_words + r) : 0ull;
            ok = ok && (idx >= n || static_cast<uint32_t>(v[u] >> 32) == call);
          }
          if (__all(ok)) break;
          if (spins == kPollLimit) {
            if (l == 0) __hip_atomic_fetch_or(a.err, 4, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
  #pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int idx = base + u * 64 + l;
          if (idx < n) {
            const int cc = idx / per_col, r = idx - cc * per_col;
            const uint32_t d = static_cast<uint32_t>(v[u]);
            if (r < a.I / 4) lds_st4_nw(hb + cc * IP + 4 * r, d);
            else lds_st1(hb + a.cb * IP + cc * kQHB + (r - a.I / 4), d);
          }
        }
      }
    }
    lds_settle_all();
    if (l == 0) lds_st4(lb + kQReady, static_cast<uint32_t>(seq + 1));
  }
}

// =================================================================== grouped form, whole-K FC1 blocks
// moe_experts_run's default.  The unit table cuts each expert's routes, in token order,
// into chunks of kChunkCols = 32 token columns (two MFMA column tiles); one weight pass
// of an expert serves a whole chunk.  One persistent, co-resident workgroup per CU:
// eight streaming waves, each with its own FC1 items, FC2 tiles and DMA ring, and a
// loader wave.
//   * an FC1 item is one hidden block of one chunk: the 64 weight rows gate 32j.. and up
//     I + 32j.. over the whole of K, against the chunk's token columns.  Items are dealt
//     round-robin over the workgroups, numbered so that the blocks of one chunk land on
//     workgroups of one XCD (whose L2 then serves the chunk's x to all of them); within a
//     workgroup, item k goes to streaming wave k mod 8, which runs all of its K steps, so
//     no FC1 partial sum leaves the wave.  The wave then applies SwiGLU and the MXFP8
//     requantization (experts page, ExpertsKernel.store_hidden) and stages the block's
//     codes and scales in LDS; the loader stores them device-coherently and raises the
//     block's flag with the call number.
//   * FC2 is dealt as 16-row output tiles, an equal contiguous run per workgroup in chunk
//     order (experts page, ExpertsKernel.partition: contiguous near-equal shares of the
//     weight stream); streaming wave w takes tiles w, w + 8, ... of the run.  The loader
//     waits for a chunk's HB flags and copies its hidden into LDS by device-coherent DMA.
//   * each streaming wave has a ring of two 8.5 KB LDS slots: an FC1 K step (four 1 KB
//     row tiles and their scale word, the x codes of the chunk's 32 columns as whole
//     lines, their scale words) or two FC2 tiles (NS2 1 KB K steps and a scale word
//     each).  A wave issues at most about one LDS DMA per 90 cycles, so eight independent
//     waves (two per SIMD) let one wave's issue overlap another's LDS reads and MFMAs.
//     Every slot is ten DMA instructions (out-of-range ones write zeros and read no
//     memory), so the wait before a slot depends only on how many of the last two slots
//     stored output rows.
constexpr int kGTiles = kChunkCols / 16;  // column tiles of a chunk
constexpr int kGStream = 8;               // streaming waves
constexpr int kGR = 2;                    // slots per streaming wave
constexpr int kGHalf = 4096 + 256;        // half a slot: four 1 KB pieces and a scale area
constexpr int kGSlot = 2 * kGHalf;
constexpr int kGOps = 10;                 // DMA instructions per slot
constexpr int kGStores = 4;               // row stores after an FC2 slot (2 tiles x 2 column tiles)
constexpr int kGLoad = kGStream;          // the loader wave
constexpr int kGWG = 64 * (kGStream + 1);
static_assert(kGLoad + 1 == kGWG / 64, "the loader is the last wave");
constexpr int kGItems = 32;               // FC1 items per workgroup (LDS token table)
constexpr int kGChunks = 1024;            // chunks per call (LDS expert table)
constexpr uint32_t kGStage = 1152;        // LDS bytes of a staged hidden block (32 x 32 codes, 32 scale words)

constexpr uint32_t kGStaged = 0;   // [kGStream] FC1 items wave w has staged
constexpr uint32_t kGPub = 32;     // [kGStream] staged items of wave w the loader has published
constexpr uint32_t kGProg2 = 64;   // [kGStream] wave w is done with every FC2 chunk sequence < value
constexpr uint32_t kGReady = 96;   // FC2 chunk sequences loaded into the hidden buffer
constexpr uint32_t kGCall = 100;   // this call's number
constexpr uint32_t kGXReady = 104; // the one-launch form: every workgroup's share of the plan is out
constexpr uint32_t kGWords = 120;  // bytes of the words above (cleared at the start)
constexpr uint32_t kGRun0 = 120;   // the three-call form: first FC2 tile of this run, posted by
constexpr uint32_t kGRun1 = 124;   // the chunk's thread before the first barrier; of the next run
constexpr uint32_t kGExp = 128;    // [kGChunks] u16 expert of chunk ch
constexpr uint32_t kGTok = kGExp + 2 * kGChunks;  // [kGItems][32] u16 pair t*K+s of item k's column (0xffff: padded)
constexpr int kGSeqMax = 8;        // chunks of a workgroup's FC2 run (the one-launch form)
constexpr uint32_t kGPairs = kGTok + 2 * kGItems * kChunkCols;  // [kGSeqMax][32] u16 pairs of the run's chunks
constexpr uint32_t kGTables = kGPairs + 2 * kGSeqMax * kChunkCols;

struct GArgs {
  const uint8_t* w13p;
  const uint8_t* s13p;
  const uint8_t* w2p;
  const uint8_t* s2p;
  const uint8_t* plan;      // x codes [B, D], then scales [B, D/32]
  const int32_t* hdr;       // unit table header (n_chunks at [4])
  const int32_t* c_expert;  // [max_chunks]
  const int32_t* c_cols;    // [max_chunks] live columns before the chunk | its live columns << 20
  const int32_t* c_pairs;   // [max_chunks][32]
  uint16_t* out;            // BF16 [B*K, D]
  uint8_t* hid;             // [max_chunks][32 columns][IP + 16]: IP code bytes, then HB scales
  uint32_t* flags;          // [max_chunks * HB] call-tagged
  uint32_t* calls;          // [kMaxGrid] per-workgroup call counters
  int32_t* err;             // status word (bit 2: a wait gave up)
  uint8_t* dump_codes;      // optional [B*K, I]
  uint8_t* dump_scales;     // optional [B*K, I/32]
  int B, K, D, I, HB, NS1, IP, floor_rule, max_chunks;
  uint64_t kinv;            // floor(2^32 / K) + 1: the token of pair p is (p kinv) >> 32, exactly (p < 2^16)
  uint32_t plan_bytes;      // bytes of the plan (x codes, then x scales)
  uint32_t out_bytes;       // bytes of the output rows
  uint32_t colb;            // bytes of one hidden column (IP + 16)
  uint32_t o_ring, o_hid, hid_code_bytes;  // LDS: rings; hidden buffer (FC1: staging), its code bytes
  // the one-launch form: the kernel makes the plan (into `plan`) and the chunk table itself
  const uint8_t* x;         // BF16 [B, D]
  const int32_t* ids;       // [B, K]
  uint32_t* pflags;         // [kMaxGrid] call-tagged: workgroup c's share of the plan is out
  int E;
};

__device__ __forceinline__ int lds_u16(uint32_t addr) {
  return static_cast<int>(lds_ld2(addr) & 0xffffu);
}

// FC1 item i -> (chunk, hidden block).  The HB items of a chunk get indices congruent mod
// 8, so that with item i dealt to workgroup i mod grid they run on workgroups of one XCD
// (workgroup c runs on XCD c mod 8) and its x rows and hidden stay in one L2.  Chunks go
// in groups of 8 kGRun: residue class r takes the kGRun consecutive chunks kGRun r ..,
// and a block's items of those chunks are 8 apart, so they run at the same time.  An
// expert's chunks are consecutive, so the chunks of an expert with more than 32 routes
// mostly stream the same weights on one XCD at once, the second read served by L2.  The
// chunks left over form groups of eight (one chunk per class); the last, partial group
// is interleaved.
constexpr int kGRun = 4;
__host__ __device__ inline void g_item(int i, int n_chunks, int HB, int& ch, int& j) {
  const int span = 8 * kGRun;
  const int big = n_chunks / span * span;          // chunks in groups of 8 kGRun
  const int small = (n_chunks - big) / 8 * 8;      // then in groups of eight
  const int i_big = big * HB, i_small = i_big + small * HB;
  if (i < i_big) {
    const int g = i / (span * HB), r = i - g * span * HB;
    const int t = r >> 3;  // r = 8 (kGRun j + s) + class
    j = t / kGRun;
    ch = span * g + kGRun * (r & 7) + (t - j * kGRun);
  } else if (i < i_small) {
    const int i1 = i - i_big, g = i1 / (8 * HB), r = i1 - g * 8 * HB;
    j = r >> 3;
    ch = big + 8 * g + (r & 7);
  } else {
    const int rem = n_chunks - big - small, i2 = i - i_small;
    j = i2 / rem;
    ch = big + small + (i2 - j * rem);
  }
}

// The grouped form's split of a launch (callable on the host too): FC1 items i = c + k *
// grid (each a whole hidden block of one chunk), and FC2 tiles in equal contiguous runs
// in chunk order (every workgroup's FC1 items run side by side in its waves, so all
// finish at about the same time).
__host__ __device__ inline QWork g_work(int n_chunks, int HB, int NS1, int D, int nwg, int c) {
  QWork q;
  q.nwg = nwg;
  q.c = c;
  q.TPE = D / 16;
  q.m1 = NS1;
  const int N1 = n_chunks * HB, N2 = n_chunks * q.TPE, cap = (N2 + nwg - 1) / nwg;
  q.n1 = N1 / nwg + (c < N1 % nwg ? 1 : 0);
  q.first2 = c * cap < N2 ? c * cap : N2;
  q.n2 = N2 - q.first2 < cap ? N2 - q.first2 : cap;
  return q;
}

// FC2 runs balanced on the bytes a tile moves (the three-call form, whose unit table
// lists each chunk's live columns and the live columns before it): its weights, 16 rows x
// (I/2 + I/32) bytes, and its output rows, 16 x 2 bytes per live column.  In units of 16
// bytes a tile of chunk ch costs u = 17 I / 32 + 2 n_ch, and the chunks before ch cost
// S(ch) = TPE (17 I / 32 ch + 2 P(ch)), P(ch) = the live columns before ch.  Workgroup c's
// run starts at the first tile whose start S(ch) + o u is at least floor(W c / grid), W =
// S(n_chunks), so the runs are contiguous, in chunk order, and cover every tile once.
// W < 2^31 for every shape the grouped kernel takes (TPE <= 1024, I <= 384, <= 1024
// chunks, <= 65536 columns), so all of it is 32-bit.
__host__ __device__ inline uint32_t g_cost_before(int ch, int prefix_cols, int TPE, int I) {
  return static_cast<uint32_t>(TPE) * (static_cast<uint32_t>(17 * I / 32) * ch + 2u * prefix_cols);
}
__host__ __device__ inline uint32_t g_run_target(uint32_t W, int t, int nwg) {
  const uint32_t q = W / nwg, r = W - q * nwg;
  return q * t + r * t / nwg;  // floor(W t / nwg), r t < 2^16
}
// The run start for target `tgt` in chunk ch (S(ch) <= tgt < S(ch + 1)).
__host__ __device__ inline int g_run_start(uint32_t tgt, uint32_t s_lo, int ncols, int ch, int TPE, int I) {
  const uint32_t u = 17u * I / 32u + 2u * ncols;
  return ch * TPE + static_cast<int>((tgt - s_lo + u - 1u) / u);
}
// Host form (schedule checks): the run of workgroup c from the chunks' live columns.
inline void g_run_host(const int32_t* ncols, int n_chunks, int D, int I, int nwg, int c, int& first, int& n2) {
  const int TPE = D / 16;
  int P = 0;
  for (int ch = 0; ch < n_chunks; ++ch) P += ncols[ch];
  const uint32_t W = g_cost_before(n_chunks, P, TPE, I);
  int t0 = 0, t1 = n_chunks * TPE;
  int pre = 0;
  for (int ch = 0; ch < n_chunks; ++ch) {
    const uint32_t lo = g_cost_before(ch, pre, TPE, I), hi = g_cost_before(ch + 1, pre + ncols[ch], TPE, I);
    const uint32_t tg0 = g_run_target(W, c, nwg), tg1 = g_run_target(W, c + 1, nwg);
    if (c > 0 && lo <= tg0 && tg0 < hi) t0 = g_run_start(tg0, lo, ncols[ch], ch, TPE, I);
    if (c + 1 < nwg && lo <= tg1 && tg1 < hi) t1 = g_run_start(tg1, lo, ncols[ch], ch, TPE, I);
    pre += ncols[ch];
  }
  first = n_chunks > 0 ? t0 : 0;
  n2 = n_chunks > 0 ? t1 - t0 : 0;
}

// Bounded LDS wait of the streaming waves.  They wait only on words that their own
// workgroup's loader posts, whose own waits are bounded, so it reads no global memory (a
// global read would wait for the wave's ring); its own bound, twice the loader's, is a
// last resort.
__device__ __forceinline__ void g_wait_lds(uint32_t addr, int want, int32_t* err) {
#pragma unroll 1
  for (uint32_t spins = 0;; ++spins) {
    if (lds_uni(addr) >= want) return;
    if (spins == 2 * kSpinLimit) {
      if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_or(err, 4, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// Bounded LDS wait of the loader: gives up (status bit 2) after kSpinLimit polls, or
// soon after another wave of the call has given up.
__device__ __forceinline__ void g_wait(uint32_t addr, int want, int32_t* err) {
#pragma unroll 1
  for (uint32_t spins = 0;; ++spins) {
    if (lds_uni(addr) >= want) return;
    if ((spins & 1023u) == 1023u) {
      const bool stop = spins >= kSpinLimit || (ld_dev_u32(err) & 4u) != 0;
      if (stop) {
        if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_or(err, 4, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
      }
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// A cursor over a streaming wave's slot sequence: the K steps of its FC1 items, then its
// FC2 tiles two per slot (tiles w, w + 8, ... of the workgroup's run), then the end.
struct GCursor {
  int k;            // slot index
  int item, si;     // FC1: the wave's item (workgroup item w + 8 * item), its K step
  int e, j, ch;     // FC1: expert, hidden block and chunk of the current item
  uint32_t xo0, xo1, xo2, xo3, xso;  // FC1 (issue side): the lane's offsets in the x code
                                     // DMAs and the x scale DMA at K step 0 (kOutside: none)
  int ti;           // FC2: the wave's tile index of the slot's first tile
  int chunk, rt2;   // FC2: chunk and 16-row tile of that tile
};

__device__ __forceinline__ void g_cursor_init(GCursor& c) {
  c.k = c.item = c.si = c.e = c.j = c.ch = c.ti = 0;
  c.xo0 = c.xo1 = c.xo2 = c.xo3 = c.xso = kOutside;
  c.chunk = c.rt2 = 0;
}

// The tile kGStream positions further in the workgroup's run.
__device__ __forceinline__ void g_next_tile(int TPE, int& chunk, int& rt2) {
  rt2 += kGStream;
#pragma unroll 1
  while (rt2 >= TPE) {
    rt2 -= TPE;
    ++chunk;
  }
}

// The x offsets of workgroup item `wi` for this lane.  The four x code DMAs of an FC1 slot
// fetch whole 128-byte lines, DMA i holding columns 8i .. 8i + 7 (eight lanes per column);
// lane l fetches part (l & 7) ^ (col & 7) of column 8i + (l >> 3), so that the slot holds
// column c's line at c * 128 with its 16-byte parts XOR-swizzled by c & 7 (the MFMA reads
// then spread over the LDS banks).  The x scale DMA fetches column l's scale word (lanes
// 0 .. 31).
__device__ __forceinline__ void g_xoffsets(const GArgs& a, uint32_t lb, int wi, uint32_t& x0, uint32_t& x1,
                                           uint32_t& x2, uint32_t& x3, uint32_t& xs) {
  const int l = threadIdx.x & 63;
  const uint32_t tb = lb + kGTok + static_cast<uint32_t>(wi * kChunkCols * 2);
  uint32_t xo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int col = 8 * i + (l >> 3);
    const int pr = lds_u16(tb + 2 * col);
    const int part = (l & 7) ^ (col & 7);
    const int t = static_cast<int>((static_cast<uint64_t>(pr) * a.kinv) >> 32);  // pr / K
    xo[i] = pr == 0xffff ? kOutside : static_cast<uint32_t>(t * a.D + 16 * part);
  }
  const int ps = l < kChunkCols ? lds_u16(tb + 2 * l) : 0xffff;
  const int ts = ps == 0xffff ? 0xffff : static_cast<int>((static_cast<uint64_t>(ps) * a.kinv) >> 32);
  x0 = xo[0];
  x1 = xo[1];
  x2 = xo[2];
  x3 = xo[3];
  xs = ts == 0xffff ? kOutside : static_cast<uint32_t>(a.B * a.D + ts * (a.D / 32));
}

// Moves the cursor to its next slot, reading the per-item state (the chunk's expert and
// the block; the issue side also the lane's x offsets) when it enters an FC1 item.  Every
// field is computed into a local and stored once (stores to different fields in
// different branches would otherwise be merged through a pointer, which puts the cursor
// in scratch memory).
__device__ __forceinline__ void g_step(const GArgs& a, const QWork& q, uint32_t lb, int w, int n1el, int n_el,
                                       int n_chunks, GCursor& c, bool tokens) {
  int k = c.k + 1, item = c.item, si = c.si, e = c.e, j = c.j, ch = c.ch, ti = c.ti;
  uint32_t xo0 = c.xo0, xo1 = c.xo1, xo2 = c.xo2, xo3 = c.xo3, xso = c.xso;
  int chunk = c.chunk, rt2 = c.rt2;
  if (c.k < n1el) {
    if (++si == a.NS1) {
      si = 0;
      ++item;
    }
  } else if (c.k < n_el) {
    ti += 2;
    g_next_tile(q.TPE, chunk, rt2);
    g_next_tile(q.TPE, chunk, rt2);
  }
  if (k < n1el && si == 0) {  // entering an FC1 item
    const int wi = w + kGStream * item;
    g_item(q.c + wi * q.nwg, n_chunks, a.HB, ch, j);
    e = __builtin_amdgcn_readfirstlane(lds_u16(lb + kGExp + 2 * ch));
    if (tokens) g_xoffsets(a, lb, wi, xo0, xo1, xo2, xo3, xso);
  } else if (k == n1el && k < n_el) {  // entering the FC2 run
    const int t = q.first2 + w;
    ti = 0;
    chunk = t / q.TPE;
    rt2 = t - chunk * q.TPE;
  }
  c.k = k;
  c.item = item;
  c.si = si;
  c.e = e;
  c.j = j;
  c.ch = ch;
  c.xo0 = xo0;
  c.xo1 = xo1;
  c.xo2 = xo2;
  c.xo3 = xo3;
  c.xso = xso;
  c.ti = ti;
  c.chunk = chunk;
  c.rt2 = rt2;
}

// Sets the cursor on slot 0 (the same per-item reads as g_step).
__device__ __forceinline__ void g_start(const GArgs& a, const QWork& q, uint32_t lb, int w, int n1el, int n_el,
                                        int n_chunks, GCursor& c, bool tokens) {
  g_cursor_init(c);
  if (0 < n1el) {
    int ch, j;
    g_item(q.c + w * q.nwg, n_chunks, a.HB, ch, j);
    c.ch = ch;
    c.j = j;
    c.e = __builtin_amdgcn_readfirstlane(lds_u16(lb + kGExp + 2 * ch));
    if (tokens) g_xoffsets(a, lb, w, c.xo0, c.xo1, c.xo2, c.xo3, c.xso);
  } else if (0 < n_el) {
    const int t = q.first2 + w;
    c.chunk = t / q.TPE;
    c.rt2 = t - c.chunk * q.TPE;
  }
}

// The x part of an FC1 slot: the chunk's 32 columns of the step as whole lines, and their
// scale words (kGOps / 2 DMA instructions).
__device__ __forceinline__ void g_issue_x(const GArgs& a, int w, const GCursor& c, __amdgpu_buffer_rsrc_t rx) {
  const uint32_t so = a.o_ring + static_cast<uint32_t>((w * kGR + c.k % kGR) * kGSlot);
  const uint32_t ks = static_cast<uint32_t>(128 * c.si);
  sdma16(rx, c.xo0, ks, so + kGHalf);
  sdma16(rx, c.xo1, ks, so + kGHalf + 1024);
  sdma16(rx, c.xo2, ks, so + kGHalf + 2048);
  sdma16(rx, c.xo3, ks, so + kGHalf + 3072);
  sdma4(rx, c.xso, static_cast<uint32_t>(4 * c.si), so + kGHalf + 4096);
}

// The slot at cursor c: always kGOps DMA instructions.  WITH_X false: an FC1 slot's
// weights only (the one-launch form's first slots, whose x part waits for the plan:
// g_issue_x then).
template <int NS2, bool WITH_X = true>
__device__ __forceinline__ void g_issue(const GArgs& a, const QWork& q, uint32_t lb, int w, int n1el, int n_el,
                                        int n2w, const GCursor& c, __amdgpu_buffer_rsrc_t rx,
                                        __amdgpu_buffer_rsrc_t none) {
  const uint32_t l = threadIdx.x & 63;
  const uint32_t v16 = 16 * l, v4 = 4 * l, vout = kOutside;
  const uint32_t so = a.o_ring + static_cast<uint32_t>((w * kGR + c.k % kGR) * kGSlot);
  if (c.k < n1el) {
    // four row tiles and their scale word (the expert's packed w13 as one buffer), then the
    // x codes of the step (the chunk's 32 columns as whole lines) and their scale words
    const int s = c.si;
    const uint32_t per = static_cast<uint32_t>(a.HB * a.NS1);  // K steps of an expert
    const uint32_t st = static_cast<uint32_t>(c.j * a.NS1 + s);
    const __amdgpu_buffer_rsrc_t rw = rsrc(a.w13p + static_cast<int64_t>(c.e) * per * 4096, per * 4096);
    const __amdgpu_buffer_rsrc_t rs = rsrc(a.s13p + static_cast<int64_t>(c.e) * per * 256, per * 256);
#pragma unroll
    for (int t = 0; t < 4; ++t) sdma16<kNT>(rw, v16, st * 4096 + t * 1024, so + t * 1024);
    sdma4<kNT>(rs, v4, st * 256, so + 4096);
    if (WITH_X) g_issue_x(a, w, c, rx);
  } else if (c.k < n_el) {
    // two FC2 tiles of the wave's sequence (the second may lie past it: nothing loaded)
    int chunk = c.chunk, rt2 = c.rt2;
    const uint32_t per = static_cast<uint32_t>(q.TPE);  // 16-row tiles of an expert
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t sh = so + h * kGHalf;
      if (c.ti + h < n2w) {
        const int e = __builtin_amdgcn_readfirstlane(lds_u16(lb + kGExp + 2 * chunk));
        const __amdgpu_buffer_rsrc_t rw = rsrc(a.w2p + static_cast<int64_t>(e) * per * NS2 * 1024, per * NS2 * 1024);
        const __amdgpu_buffer_rsrc_t rs = rsrc(a.s2p + static_cast<int64_t>(e) * per * 256, per * 256);
        const uint32_t t0 = static_cast<uint32_t>(rt2);
#pragma unroll
        for (int ks = 0; ks < NS2; ++ks) sdma16<kNT>(rw, v16, (t0 * NS2 + ks) * 1024, sh + ks * 1024);
#pragma unroll
        for (int ks = NS2; ks < 4; ++ks) sdma16(none, vout, 0, sh + ks * 1024);
        sdma4<kNT>(rs, v4, t0 * 256, sh + 4096);
      } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) sdma16(none, vout, 0, sh + ks * 1024);
        sdma4(none, vout, 0, sh + 4096);
      }
      g_next_tile(q.TPE, chunk, rt2);
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) sdma16(none, vout, 0, so + h * kGHalf + ks * 1024);
      sdma4(none, vout, 0, so + h * kGHalf + 4096);
    }
  }
}

// The BF16 row pieces of one FC2 tile, stored after the slot's refill is issued.
struct GRows {
  uint2 v0, v1;        // column tile 0 / 1: four BF16 values of the lane's output row
  uint32_t off0, off1; // their byte offsets in the output (out of range: not written)
};

__device__ __forceinline__ void g_store_rows(const GRows& r, __amdgpu_buffer_rsrc_t rout) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u, r.v0), rout, static_cast<int>(r.off0), 0, 0);
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u, r.v1), rout, static_cast<int>(r.off1), 0, 0);
}

// One FC2 tile from half a slot against the hidden of its chunk: 16 output rows x the
// chunk's two column tiles (the second skipped for a chunk of <= 16 columns).  Past the
// wave's sequence it computes nothing and both row offsets are out of range.
template <int NS2>
__device__ __forceinline__ GRows g_fc2_tile(const GArgs& a, uint32_t lb, int w, int g0, bool live_tile, int chunk,
                                            int rt2, uint32_t sh, int& seq_cur, uint32_t& hbl, uint32_t& hbs,
                                            int& orow0, int& orow1) {
  const int l = threadIdx.x & 63, grp = l >> 4, col = l & 15;
  v4f o0 = v4f{0.f, 0.f, 0.f, 0.f}, o1 = v4f{0.f, 0.f, 0.f, 0.f};
  bool second = false;
  if (live_tile) {
    const int seq = chunk - g0;
    if (seq != seq_cur) {
      seq_cur = seq;
      if (l == 0) lds_st4(lb + kGProg2 + 4 * w, static_cast<uint32_t>(seq));
      g_wait_lds(lb + kGReady, seq + 1, a.err);
      const uint32_t hb = lb + a.o_hid;
      hbl = hb + col * a.colb + 16 * grp;
      hbs = hb + col * a.colb + a.IP;
      const int p0 = static_cast<int>(lds_ld4(hb + a.hid_code_bytes + 4 * col));
      const int p1 = static_cast<int>(lds_ld4(hb + a.hid_code_bytes + 4 * (16 + col)));
      orow0 = p0 >= 0 ? p0 * a.D : -1;
      orow1 = p1 >= 0 ? p1 * a.D : -1;
    }
    uint4 wa0, wa1, wa2, wa3;
    uint32_t was;
    asm volatile(
        "ds_read_b128 %0, %5 offset:0\n\t"
        "ds_read_b128 %1, %5 offset:1024\n\t"
        "ds_read_b128 %2, %5 offset:2048\n\t"
        "ds_read_b128 %3, %5 offset:3072\n\t"
        "ds_read_b32 %4, %6 offset:4096\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(wa0), "=&v"(wa1), "=&v"(wa2), "=&v"(wa3), "=&v"(was)
        : "v"(sh + l * 16), "v"(sh + l * 4)
        : "memory");
    const uint4 wa[4] = {wa0, wa1, wa2, wa3};
    {
      HidOps<NS2> hop;
      hid_read<NS2>(hbl, hbs, hop);
      // K-blocks past I hold zero codes (weights and hidden)
#pragma unroll
      for (int s = 0; s < NS2; ++s)
        o0 = mfma_fp4_fp8(fp4_operand(wa[s]), fp8_operand(hop.bl[s], hop.bh[s]), o0,
                          static_cast<int>((was >> (8 * s)) & 0xffu), static_cast<int>((hop.bs[s] >> (8 * grp)) & 0xffu));
    }
    second = __any(orow1 >= 0);  // a chunk of <= 16 columns skips its second column tile
    if (second) {
      HidOps<NS2> hop;
      hid_read<NS2>(hbl + 16 * a.colb, hbs + 16 * a.colb, hop);
#pragma unroll
      for (int s = 0; s < NS2; ++s)
        o1 = mfma_fp4_fp8(fp4_operand(wa[s]), fp8_operand(hop.bl[s], hop.bh[s]), o1,
                          static_cast<int>((was >> (8 * s)) & 0xffu), static_cast<int>((hop.bs[s] >> (8 * grp)) & 0xffu));
    }
    mfma_settle(o0);
    mfma_settle(o1);
  }
  const uint32_t ro = static_cast<uint32_t>(16 * rt2 + 4 * grp) * 2;
  GRows r;
  r.off0 = live_tile && orow0 >= 0 ? static_cast<uint32_t>(orow0) * 2 + ro : kOutside;
  r.off1 = live_tile && second && orow1 >= 0 ? static_cast<uint32_t>(orow1) * 2 + ro : kOutside;
  r.v0 = make_uint2(bf16_pair(o0[0], o0[1]), bf16_pair(o0[2], o0[3]));
  r.v1 = make_uint2(bf16_pair(o1[0], o1[1]), bf16_pair(o1[2], o1[3]));
  return r;
}

// SwiGLU and MXFP8 of a finished FC1 item (experts page, store_hidden), staged in LDS at
// `stg` for the loader: column c's 32 codes at c * 32, its scale (E8M0 byte, as a word) at
// 1024 + 4c.  Lane
// (col, grp) holds hidden values 32j + 4grp + r (row tile 0 over 1) and 32j + 16 + 4grp + r
// of column col of each column tile.
__device__ __forceinline__ void g_finish(const GArgs& a, v4f (&acc)[4][kGTiles], int ncc, uint32_t stg) {
  const int l = threadIdx.x & 63, grp = l >> 4, col = l & 15;
#pragma unroll
  for (int cc = 0; cc < kGTiles; ++cc) {
    if (cc >= ncc) continue;
    float h[2][4];
    float amax = 0.0f;
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float gv = acc[half][cc][r], uv = acc[2 + half][cc][r];
        // SwiGLU with the hardware exponential and reciprocal (a few ulp in FP32; the
        // hidden is then rounded to 3 mantissa bits)
        h[half][r] = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
        amax = fmaxf(amax, fabsf(h[half][r]));
      }
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    const int e = mx_exponent(amax, a.floor_rule != 0);
    const float sc = exp2_neg(e);
    auto clampf = [](float v) { return fminf(fmaxf(v, -448.0f), 448.0f); };  // the floor rule saturates
    uint32_t word[2];
#pragma unroll
    for (int half = 0; half < 2; ++half)
      word[half] = cvt4_e4m3(clampf(h[half][0] * sc), clampf(h[half][1] * sc), clampf(h[half][2] * sc),
                             clampf(h[half][3] * sc));
    const uint32_t cl = static_cast<uint32_t>(cc * 16 + col);
    lds_st4(stg + cl * 32 + 4 * grp, word[0]);
    lds_st4(stg + cl * 32 + 16 + 4 * grp, word[1]);
    if (grp == 0) lds_st4(stg + 1024 + 4 * cl, static_cast<uint32_t>(e + 127));
  }
}

// ------------------------------------------ the grouped form in one launch (prologue)
// The one-launch form's prologue, in every workgroup: (1) its share of the MXFP8 plan of
// x (experts page, plan_chunk / mx_block; four lanes per 32-element block), stored
// device-coherent and published with a call-tagged flag; (2) the chunk table of the batch
// (experts page, ExpertsGroupKernel: each expert's routes in token order, cut into chunks
// of 32), built in LDS from the ids -- per-expert token bitmasks, route counts, an
// exclusive scan of the chunk counts -- using `scr`, LDS no DMA has reached yet; then one
// more pass over the routes places each route of a chunk this workgroup needs (its FC1
// items' and its FC2 run's) at its rank.  It leaves the chunks' experts in kGExp, the
// pairs of its FC1 items in kGTok and those of its FC2 run in kGPairs, and returns the
// chunk count (uniform).
__device__ __forceinline__ int g_fused_prologue(const GArgs& a, uint32_t scr, uint32_t call, bool& x_early) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ uint32_t wsum[kGWG / 64];
  __shared__ int s_flags, s_total;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nwg = gridDim.x, c = blockIdx.x;
  const int E = a.E, K = a.K, U = a.B * K, W = (a.B + 31) / 32;
  // the routes, requested first (they arrive while the plan share is made)
  constexpr int kHeld = 8;  // routes held in registers per thread (all of them for U <= 4608)
  int ev[kHeld];
#pragma unroll
  for (int h = 0; h < kHeld; ++h) ev[h] = tid + h * kGWG < U ? a.ids[tid + h * kGWG] : -1;
  // the plan share: 32-element blocks [c nb / grid, (c + 1) nb / grid), four lanes per
  // block; the first quarter of each lane is requested with the routes
  const int64_t nb = static_cast<int64_t>(a.B) * a.D / 32;
  const int64_t b0 = nb * c / nwg, b1 = nb * (c + 1) / nwg, q0 = 4 * b0 + tid;
  uint4 xq = ld16(a.x + (q0 < 4 * b1 ? q0 : 0) * 16);  // unconditional: no select waits for it
  compiler_fence();  // the load stays ahead of the LDS set-up below
  // (2) the chunk table's LDS, set up while the loads are in flight
  uint32_t* masks = reinterpret_cast<uint32_t*>(smem + scr);  // [W][E]
  int* routes = reinterpret_cast<int*>(masks + W * E);        // [E] route counts, then token counts
  int* chunk0 = routes + E;                                   // [E] first chunk
  int* slot = chunk0 + E;                                     // [kGChunks] the chunk's row of `rows`
  uint16_t* rows = reinterpret_cast<uint16_t*>(slot + kGChunks);  // [kGItems + kGSeqMax][32] pairs
  for (int i = tid; i < W * E; i += kGWG) masks[i] = 0u;
  for (int i = tid; i < E; i += kGWG) routes[i] = 0;
  for (int i = tid; i < kGChunks; i += kGWG) slot[i] = 0x7fffffff;
  for (int i = tid; i < (kGItems + kGSeqMax) * kChunkCols; i += kGWG) rows[i] = 0xffff;
  if (tid == 0) s_flags = 0;
  // (1) the plan share.  The held routes and the first x quarter pass through an empty
  // asm first: one wait for all of them, before any store, so that no later use of the
  // routes waits for the plan's stores, which drain while the routes are marked (the
  // share's flag goes out after that)
#pragma unroll
  for (int h = 0; h < kHeld; ++h) asm volatile("" : "+v"(ev[h]));
  asm volatile("" : "+v"(xq.x), "+v"(xq.y), "+v"(xq.z), "+v"(xq.w));
  {
    uint8_t* codes = const_cast<uint8_t*>(a.plan);
    uint8_t* scales = codes + static_cast<int64_t>(a.B) * a.D;
    if (q0 < 4 * b1) plan_quarter_dev_v(xq, q0, codes, scales);
    for (int64_t idx4 = q0 + kGWG; idx4 < 4 * b1; idx4 += kGWG) plan_quarter_dev(a.x, idx4, codes, scales);
  }
  __syncthreads();
  int bad = 0;
  // the token of route r, r / K, as a multiply-high: exact, since the error of kinv is
  // below 2^-32 K and r < 2^16
  const uint64_t kinv = a.kinv;
  auto token = [&](int r) { return static_cast<int>((static_cast<uint64_t>(r) * kinv) >> 32); };
  auto mark = [&](int r, int e) {
    if (e < 0 || e >= E) {
      bad = 1;
      return;
    }
    const int t = token(r);
    atomicOr(&masks[(t >> 5) * E + e], 1u << (t & 31));
    atomicAdd(&routes[e], 1);
  };
#pragma unroll
  for (int h = 0; h < kHeld; ++h)
    if (tid + h * kGWG < U) mark(tid + h * kGWG, ev[h]);
  for (int r = tid + kHeld * kGWG; r < U; r += kGWG) mark(r, a.ids[r]);
  if (bad) atomicOr(&s_flags, 1);
  wait_stores();  // every lane's device-coherent plan stores are done ...
  __syncthreads();
  if (tid == 0) st_dev_u32(a.pflags + c, call);  // ... before the share's flag
  // thread i holds experts 2i and 2i + 1: their token counts and chunk counts, scanned
  int cnt[2], nch[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int e = 2 * tid + h;
    cnt[h] = 0;
    if (e < E) {
      for (int wd = 0; wd < W; ++wd) cnt[h] += __popc(masks[wd * E + e]);
      if (cnt[h] != routes[e]) atomicOr(&s_flags, 2);  // an id repeated within a token
    }
    nch[h] = (cnt[h] + kChunkCols - 1) / kChunkCols;
  }
  const uint32_t local = static_cast<uint32_t>(nch[0] + nch[1]);
  const uint32_t incl = wave_scan_u32(local);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t before = 0;
  for (int wv = 0; wv < wave; ++wv) before += wsum[wv];
  if (tid == kGWG - 1) s_total = static_cast<int>(before + incl);
  const int first = static_cast<int>(before + incl - local);
  // the chunk entries of this thread's experts (after every count is read)
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int e = 2 * tid + h;
    if (e < E) {
      const int c0 = first + (h ? nch[0] : 0);
      routes[e] = 0;  // from here on: 1 when a chunk of e is needed here
      chunk0[e] = c0;
      for (int q = 0; q < nch[h] && c0 + q < kGChunks; ++q) reinterpret_cast<uint16_t*>(smem + kGExp)[c0 + q] = static_cast<uint16_t>(e);
    }
  }
  __syncthreads();
  const int n_chunks = s_total;
  if (c == 0 && tid == 0 && s_flags != 0) __hip_atomic_fetch_or(a.err, s_flags, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // the chunks this workgroup needs, its FC1 items' (k < n1) and its FC2 run's (k = n1 +
  // sequence): each chunk's row of `rows` is the least k that needs it
  const QWork q = g_work(n_chunks, a.HB, a.NS1, a.D, nwg, c);
  const int n1 = q.n1 < kGItems ? q.n1 : kGItems;
  const int g0 = q.first2 / q.TPE;
  int nseq = q.n2 > 0 ? (q.first2 + q.n2 - 1) / q.TPE - g0 + 1 : 0;
  nseq = nseq < kGSeqMax ? nseq : kGSeqMax;
  int my_ch = n_chunks;  // the chunk of k = tid
  if (tid < n1 + nseq) {
    int jj;
    my_ch = g0 + tid - n1;
    if (tid < n1) g_item(c + tid * nwg, n_chunks, a.HB, my_ch, jj);
    if (my_ch < n_chunks) {
      atomicMin(&slot[my_ch], tid);
      routes[reinterpret_cast<const uint16_t*>(smem + kGExp)[my_ch]] = 1;
    }
  }
  __syncthreads();
  // every route of a needed chunk, at its rank: its position among its expert's routes in
  // token order (the token bits below it)
  auto needed = [&](int e) { return e >= 0 && e < E && routes[e] != 0; };  // a chunk of e is needed here
  auto place = [&](int r, int e) {
    const int t = token(r), tw = t >> 5;
    int rank = __popc(masks[tw * E + e] & ((1u << (t & 31)) - 1u));
    for (int wd = 0; wd < tw; ++wd) rank += __popc(masks[wd * E + e]);
    const int sl = slot[chunk0[e] + rank / kChunkCols];
    if (sl < kGItems + kGSeqMax) rows[sl * kChunkCols + rank % kChunkCols] = static_cast<uint16_t>(r);
  };
  // a lane's held routes that are needed, then one of them per pass: the wave makes as
  // many passes as its busiest lane has such routes (few: a workgroup needs the chunks of
  // a handful of experts), not one per held route
  uint32_t todo = 0;
#pragma unroll
  for (int h = 0; h < kHeld; ++h)
    if (tid + h * kGWG < U && needed(ev[h])) todo |= 1u << h;
  // the loader wave asks early whether every workgroup's plan share is out; the answer is
  // read after the placement.  The held routes pass through an empty asm first, so that
  // no later use of them waits for a load (a wait for them would also wait for these).
#pragma unroll
  for (int h = 0; h < kHeld; ++h) asm volatile("" : "+v"(ev[h]));
  uint32_t pf[4] = {0u, 0u, 0u, 0u};
  if (wave == kGStream) {
#pragma unroll
    for (int i = 0; i < 4; ++i) pf[i] = ld_dev_u32(a.pflags + min(lane + 64 * i, nwg - 1));  // no branch
  }
#pragma unroll 1
  while (__any(todo != 0)) {
    if (todo != 0) {
      const int hn = __ffs(todo) - 1;
      todo &= todo - 1u;
      int e = 0;
#pragma unroll
      for (int h = 0; h < kHeld; ++h) e = h == hn ? ev[h] : e;
      place(tid + hn * kGWG, e);
    }
  }
  for (int r = tid + kHeld * kGWG; r < U; r += kGWG) {
    const int e = a.ids[r];
    if (needed(e)) place(r, e);
  }
  __syncthreads();
  // row k of the tables: the row of thread k's chunk, shared through LDS
  int* kch = reinterpret_cast<int*>(rows + (kGItems + kGSeqMax) * kChunkCols);  // [kGItems + kGSeqMax]
  if (tid < n1 + nseq) kch[tid] = my_ch < n_chunks ? slot[my_ch] : -1;
  __syncthreads();
  for (int idx = tid; idx < (n1 + nseq) * kChunkCols; idx += kGWG) {
    const int k = idx / kChunkCols, cl = idx - k * kChunkCols;
    const int row = kch[k];
    const uint16_t v = row >= 0 ? rows[row * kChunkCols + cl] : static_cast<uint16_t>(0xffff);
    if (k < n1) reinterpret_cast<uint16_t*>(smem + kGTok)[idx] = v;
    else reinterpret_cast<uint16_t*>(smem + kGPairs)[idx - n1 * kChunkCols] = v;
  }
  if (wave == kGStream) {
    bool ok = nwg <= 256;
#pragma unroll
    for (int i = 0; i < 4; ++i) ok = ok && (lane + 64 * i >= nwg || pf[i] == call);
    x_early = __all(ok);
  }
  __syncthreads();
  return n_chunks;
}

template <int NS2, bool FUSED>
__global__ __launch_bounds__(kGWG) void grouped_kernel(GArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  agpr_form();
  const int tid = threadIdx.x, l = tid & 63, w = wave_id();
  const int grp = l >> 4, col = l & 15;
  const uint32_t lb = lds_base();
  const int nwg = gridDim.x, c = blockIdx.x;
  const int HB = a.HB, NS1 = a.NS1;
  uint32_t* sw = reinterpret_cast<uint32_t*>(smem);

  // ---- prologue: the chunk count, the chunks' experts and the pair columns of this
  // workgroup's FC1 items, all requested at once (read for every possible chunk: the
  // table holds max_chunks records, and the item numbering depends on the chunk count);
  // the one-launch form makes them, and its share of the plan, itself
  if (tid < static_cast<int>(kGWords / 4)) sw[tid] = 0u;
  int n_chunks = 0;
  bool x_early = false;  // the one-launch form's loader: every plan share was out already
  if constexpr (FUSED) {
    if (tid == 0) sw[kGCall / 4] = ld_dev_u32(a.calls + c) + 1u;  // stored back at the end
    __syncthreads();
    n_chunks = g_fused_prologue(a, a.o_ring, sw[kGCall / 4], x_early);
  } else {
    n_chunks = a.hdr[4];
    const int n1_cap = (n_chunks * HB - c + nwg - 1) / nwg;  // this workgroup's FC1 items
    static_assert(kGChunks <= 2 * kGWG && kGItems * kChunkCols <= 2 * kGWG, "two entries a thread");
    // loads first: two chunk records a thread, then two pair columns of the items (their
    // addresses need the chunk count)
    int ex[2], cc[2], pr[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ch = tid + i * kGWG;
      const bool v = ch < a.max_chunks && ch < kGChunks;
      ex[i] = v ? a.c_expert[ch] : 0;
      cc[i] = v ? a.c_cols[ch] : 0;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + i * kGWG;
      pr[i] = -1;
      if (idx < n1_cap * kChunkCols && idx < kGItems * kChunkCols) {
        const int k = idx / kChunkCols, cl = idx - k * kChunkCols;
        int ch, jj;
        g_item(c + k * nwg, n_chunks, HB, ch, jj);
        pr[i] = a.c_pairs[static_cast<int64_t>(ch) * kChunkCols + cl];
      }
    }
    // the byte-balanced FC2 runs (g_run_start): the thread of the chunk that holds this
    // run's start, and the next run's, posts it
    const int TPE = a.D / 16;
    const uint32_t W = g_cost_before(n_chunks, a.hdr[5], TPE, a.I);
    const uint32_t tgt0 = g_run_target(W, c, nwg), tgt1 = g_run_target(W, c + 1, nwg);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ch = tid + i * kGWG;
      const int p0 = cc[i] & 0xfffff, nc = cc[i] >> 20;
      if (ch < n_chunks) {
        const uint32_t lo = g_cost_before(ch, p0, TPE, a.I), hi = g_cost_before(ch + 1, p0 + nc, TPE, a.I);
        if (lo <= tgt0 && tgt0 < hi) sw[kGRun0 / 4] = static_cast<uint32_t>(g_run_start(tgt0, lo, nc, ch, TPE, a.I));
        if (lo <= tgt1 && tgt1 < hi) sw[kGRun1 / 4] = static_cast<uint32_t>(g_run_start(tgt1, lo, nc, ch, TPE, a.I));
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ch = tid + i * kGWG, idx = tid + i * kGWG;
      if (ch < a.max_chunks && ch < kGChunks) reinterpret_cast<uint16_t*>(smem + kGExp)[ch] = static_cast<uint16_t>(ex[i]);
      if (idx < n1_cap * kChunkCols && idx < kGItems * kChunkCols)
        reinterpret_cast<uint16_t*>(smem + kGTok)[idx] = static_cast<uint16_t>(pr[i] >= 0 ? pr[i] : 0xffff);
    }
    if (tid == 0) sw[kGCall / 4] = ld_dev_u32(a.calls + c) + 1u;  // stored back at the end
    __syncthreads();
  }

  QWork q = g_work(n_chunks, HB, NS1, a.D, nwg, c);
  if constexpr (!FUSED) {
    // run c starts at tile 0 for c = 0 and the last ends at the last tile; no chunk, no run
    const int N2 = n_chunks * q.TPE;
    const int t0 = c == 0 ? 0 : static_cast<int>(sw[kGRun0 / 4]);
    const int t1 = c + 1 == nwg ? N2 : static_cast<int>(sw[kGRun1 / 4]);
    q.first2 = n_chunks > 0 ? t0 : 0;
    q.n2 = n_chunks > 0 ? t1 - t0 : 0;
  }
  const int g0 = q.first2 / q.TPE;  // chunk of the workgroup's first FC2 tile (sequence 0)
  const __amdgpu_buffer_rsrc_t none =
      __builtin_amdgcn_make_buffer_rsrc(static_cast<void*>(a.out), static_cast<short>(0), 0u, 0x00020000);

  if (w < kGStream) {
    // =============================================================== streaming wave
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.plan), static_cast<short>(0), static_cast<int>(a.plan_bytes), 0x00020000);
    const __amdgpu_buffer_rsrc_t rout = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<void*>(a.out), static_cast<short>(0), static_cast<int>(a.out_bytes), 0x00020000);
    const int n1w = q.n1 > w ? (q.n1 - w + kGStream - 1) / kGStream : 0;  // the wave's FC1 items
    const int n1el = n1w * NS1;
    const int n2w = q.n2 > w ? (q.n2 - w + kGStream - 1) / kGStream : 0;  // the wave's FC2 tiles
    const int n_el = n1el + (n2w + 1) / 2;                                 // two per slot
    const uint32_t stg = lb + a.o_hid + static_cast<uint32_t>(w) * kGStage;  // the wave's staging
    GCursor ic, cs;  // issue side (two slots ahead), consume side
    g_start(a, q, lb, w, n1el, n_el, n_chunks, ic, true);
    g_start(a, q, lb, w, n1el, n_el, n_chunks, cs, false);
    static_assert(kGR == 2 && kGOps == 10, "the wait counts below assume two slots of ten");
    // the one-launch form: the first two slots' weights now, their x once the whole plan is
    // out (both slots are FC1 steps of the wave's first item: an item has NS1 >= 2 steps)
    const bool split = FUSED && n1el > 0;
    if (split) {
      GCursor c0 = ic;
      g_issue<NS2, false>(a, q, lb, w, n1el, n_el, n2w, ic, rx, none);
      g_step(a, q, lb, w, n1el, n_el, n_chunks, ic, true);
      GCursor c1 = ic;
      g_issue<NS2, false>(a, q, lb, w, n1el, n_el, n2w, ic, rx, none);
      g_step(a, q, lb, w, n1el, n_el, n_chunks, ic, true);
      g_wait_lds(lb + kGXReady, 1, a.err);
      g_issue_x(a, w, c0, rx);
      g_issue_x(a, w, c1, rx);
    } else {
#pragma unroll 1
      for (int p = 0; p < kGR; ++p) {
        g_issue<NS2>(a, q, lb, w, n1el, n_el, n2w, ic, rx, none);
        g_step(a, q, lb, w, n1el, n_el, n_chunks, ic, true);
      }
    }
    v4f acc[4][kGTiles];
    const uint32_t xq_lo = static_cast<uint32_t>(col * 128 + 16 * (grp ^ (col & 7)));
    int ncc = 1, seq_cur = -1;
    uint32_t hbl = 0, hbs = 0;
    int orow0 = -1, orow1 = -1;
#pragma unroll 1
    for (int k = 0; k < n_el; ++k) {
      // slot k has landed: younger are the next slot and the row stores of the last two
      // consumed slots (kGStores after each FC2 slot)
      const int nf = k - n1el < 0 ? 0 : (k - n1el > 2 ? 2 : k - n1el);
      if (split && k == 0) wait_vm<kGOps / 2>();  // younger: slot 1's x part only
      else if (nf == 0) wait_vm<kGOps>();
      else if (nf == 1) wait_vm<kGOps + kGStores>();
      else wait_vm<kGOps + 2 * kGStores>();
      const uint32_t sa = lb + a.o_ring + static_cast<uint32_t>((w * kGR + k % kGR) * kGSlot);
      if (k < n1el) {
        // ---- FC1 step: four row tiles x the chunk's column tiles
        if (cs.si == 0) {
          const int wi = w + kGStream * cs.item;
          ncc = lds_u16(lb + kGTok + static_cast<uint32_t>((wi * kChunkCols + 16) * 2)) == 0xffff ? 1 : 2;
          ncc = __builtin_amdgcn_readfirstlane(ncc);
#pragma unroll
          for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int cc = 0; cc < kGTiles; ++cc) acc[rt][cc] = v4f{0.f, 0.f, 0.f, 0.f};
        }
        // x codes of column col: K 16 grp.. (part grp) and 64 + 16 grp.. (part 4 + grp) of its
        // swizzled line, and its scale word of the step; both column tiles with one wait (for
        // a chunk of <= 16 columns the second is zeros and unused)
        const uint32_t sb = sa + kGHalf;
        const uint32_t xlo = sb + xq_lo, xhi = sb + (xq_lo ^ 64u);
        uint4 a0, a1, a2, a3, xl, xh, yl, yh;
        uint32_t as, xs, ys;
        asm volatile(
            "ds_read_b128 %0, %11 offset:0\n\t"
            "ds_read_b128 %1, %11 offset:1024\n\t"
            "ds_read_b128 %2, %11 offset:2048\n\t"
            "ds_read_b128 %3, %11 offset:3072\n\t"
            "ds_read_b32 %4, %12 offset:4096\n\t"
            "ds_read_b128 %5, %13 offset:0\n\t"
            "ds_read_b128 %6, %14 offset:0\n\t"
            "ds_read_b32 %7, %15 offset:4096\n\t"
            "ds_read_b128 %8, %13 offset:2048\n\t"
            "ds_read_b128 %9, %14 offset:2048\n\t"
            "ds_read_b32 %10, %15 offset:4160\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3), "=&v"(as), "=&v"(xl), "=&v"(xh), "=&v"(xs), "=&v"(yl),
              "=&v"(yh), "=&v"(ys)
            : "v"(sa + l * 16), "v"(sa + l * 4), "v"(xlo), "v"(xhi), "v"(sb + col * 4)
            : "memory");
        const uint4 av[4] = {a0, a1, a2, a3};
        {
          const v8i b = fp8_operand(xl, xh);
          const int sbv = static_cast<int>((xs >> (8 * grp)) & 0xffu);
#pragma unroll
          for (int rt = 0; rt < 4; ++rt)
            acc[rt][0] = mfma_fp4_fp8(fp4_operand(av[rt]), b, acc[rt][0], static_cast<int>((as >> (8 * rt)) & 0xffu), sbv);
        }
        if (ncc > 1) {
          const v8i b = fp8_operand(yl, yh);
          const int sbv = static_cast<int>((ys >> (8 * grp)) & 0xffu);
#pragma unroll
          for (int rt = 0; rt < 4; ++rt)
            acc[rt][1] = mfma_fp4_fp8(fp4_operand(av[rt]), b, acc[rt][1], static_cast<int>((as >> (8 * rt)) & 0xffu), sbv);
        }
        // refill the slot just consumed (two slots ahead)
        g_issue<NS2>(a, q, lb, w, n1el, n_el, n2w, ic, rx, none);
        g_step(a, q, lb, w, n1el, n_el, n_chunks, ic, true);
        if (cs.si == NS1 - 1) {
          // the item is done: SwiGLU and MXFP8 into the wave's staging area, once the loader
          // has published the wave's previous item from it
#pragma unroll
          for (int cc = 0; cc < kGTiles; ++cc) mfma_settle(acc[0][cc], acc[1][cc], acc[2][cc], acc[3][cc]);
          g_wait_lds(lb + kGPub + 4 * w, cs.item, a.err);
          g_finish(a, acc, ncc, stg);
          if (l == 0) lds_st4(lb + kGStaged + 4 * w, static_cast<uint32_t>(cs.item + 1));
        }
      } else {
        // ---- two FC2 tiles, computed before the refill overwrites the slot; the refill
        // is issued first, then the four row stores
        const int ti = cs.ti, chunk0 = cs.chunk, rt20 = cs.rt2;
        int chunk1 = chunk0, rt21 = rt20;
        g_next_tile(q.TPE, chunk1, rt21);
        const GRows r0 = g_fc2_tile<NS2>(a, lb, w, g0, ti < n2w, chunk0, rt20, sa, seq_cur, hbl, hbs, orow0, orow1);
        const GRows r1 =
            g_fc2_tile<NS2>(a, lb, w, g0, ti + 1 < n2w, chunk1, rt21, sa + kGHalf, seq_cur, hbl, hbs, orow0, orow1);
        g_issue<NS2>(a, q, lb, w, n1el, n_el, n2w, ic, rx, none);
        g_step(a, q, lb, w, n1el, n_el, n_chunks, ic, true);
        g_store_rows(r0, rout);
        g_store_rows(r1, rout);
      }
      g_step(a, q, lb, w, n1el, n_el, n_chunks, cs, false);
    }
    if (l == 0) lds_st4(lb + kGProg2 + 4 * w, 0x7fffffffu);
    wait_vm<0>();  // the dummy slots land before the wave ends
    return;
  }

  // ================================================================= loader wave
  const uint32_t call = static_cast<uint32_t>(lds_uni(lb + kGCall));
  if constexpr (FUSED) {
    // the one-launch form: wait until every workgroup's share of the plan is out, then
    // acquire (the L2 and L1 drop what they held of the plan's lines) before the streaming
    // waves read x
#pragma unroll 1
    for (uint32_t spins = 0; !x_early; ++spins) {
      bool ok = true;
      for (int i = l; i < nwg; i += 64) ok = ok && ld_dev_u32(a.pflags + i) == call;
      if (__all(ok)) break;
      if (poll_expired(spins, a.err)) {
        if (l == 0) __hip_atomic_fetch_or(a.err, 4, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    wait_vm<0>();
    if (l == 0) lds_st4(lb + kGXReady, 1u);
  }
  // FC1: publish the staged hidden blocks in the workgroup's item order (item k is wave
  // k mod 8's (k / 8)-th): codes and scale of each column (device-coherent stores), then
  // the block's flag with the call number.  The items found staged together (the waves
  // tend to finish theirs at the same time) go out under one wait for their stores; a
  // wave may refill its staging area once the loader has read it.
#pragma unroll 1
  for (int k = 0; k < q.n1;) {
    g_wait(lb + kGStaged + 4 * (k % kGStream), k / kGStream + 1, a.err);
    int k1 = k + 1;  // one past the batch
#pragma unroll 1
    while (k1 < q.n1 && lds_uni(lb + kGStaged + 4 * (k1 % kGStream)) >= k1 / kGStream + 1) ++k1;
#pragma unroll 1
    for (int kk = k; kk < k1; ++kk) {
      const int ww = kk % kGStream, m = kk / kGStream;
      int ch, j;
      g_item(c + kk * nwg, n_chunks, HB, ch, j);
      const uint32_t stg = lb + a.o_hid + static_cast<uint32_t>(ww) * kGStage;
      const int cl = l >> 1, part = l & 1;  // lane: 16 code bytes of column cl
      const uint4 v = lds_ld16(stg + static_cast<uint32_t>(cl * 32 + 16 * part));
      const uint32_t sc = lds_ld4(stg + 1024 + 4 * static_cast<uint32_t>(cl));
      if (l == 0) lds_st4(lb + kGPub + 4 * ww, static_cast<uint32_t>(m + 1));  // after the reads (in order)
      uint8_t* dst = a.hid + (static_cast<int64_t>(ch) * kChunkCols + cl) * a.colb;
      st_dev_u64(dst + 32 * j + 16 * part, static_cast<uint64_t>(v.x) | (static_cast<uint64_t>(v.y) << 32));
      st_dev_u64(dst + 32 * j + 16 * part + 8, static_cast<uint64_t>(v.z) | (static_cast<uint64_t>(v.w) << 32));
      if (part == 0) st_dev_u8(dst + a.IP + j, static_cast<uint8_t>(sc));
      if (a.dump_codes != nullptr) {
        const int pair = kk < kGItems ? lds_u16(lb + kGTok + static_cast<uint32_t>((kk * kChunkCols + cl) * 2)) : 0xffff;
        if (pair != 0xffff) {
          *reinterpret_cast<uint4*>(a.dump_codes + static_cast<int64_t>(pair) * a.I + 32 * j + 16 * part) = v;
          if (part == 0) a.dump_scales[static_cast<int64_t>(pair) * HB + j] = static_cast<uint8_t>(sc);
        }
      }
    }
    wait_stores();
#pragma unroll 1
    for (int kk = k; kk < k1; ++kk) {
      int ch, j;
      g_item(c + kk * nwg, n_chunks, HB, ch, j);
      if (l == 0) st_dev_u32(a.flags + static_cast<int64_t>(ch) * HB + j, call);
    }
    k = k1;
  }
  // FC2: for each chunk of the workgroup's run, in order: wait for its HB block flags,
  // then copy its hidden (codes and scales, device-coherent DMA) and its columns' pair
  // indices into the LDS hidden buffer (which held the staging areas during FC1), once
  // every streaming wave is done with the previous chunk.
  const int nseq = q.n2 > 0 ? (q.first2 + q.n2 - 1) / q.TPE - g0 + 1 : 0;
#pragma unroll 1
  for (int seq = 0; seq < nseq; ++seq) {
    const int ch = g0 + seq;
    if (seq >= 1) {
#pragma unroll 1
      for (int ww = 0; ww < kGStream; ++ww) g_wait(lb + kGProg2 + 4 * ww, seq, a.err);
    }
    const uint32_t* f = a.flags + static_cast<int64_t>(ch) * HB;
#pragma unroll 1
    for (uint32_t spins = 0;; ++spins) {
      const bool ok = l >= HB || ld_dev_u32(f + l) == call;
      if (__all(ok)) break;
      if (poll_expired(spins, a.err)) {
        if (l == 0) __hip_atomic_fetch_or(a.err, 4, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    compiler_fence();
    const uint32_t hb = a.o_hid;  // offset from smem
    const uint8_t* src = a.hid + static_cast<int64_t>(ch) * kChunkCols * a.colb;
    for (uint32_t off = 0; off < a.hid_code_bytes; off += 1024)
      __builtin_amdgcn_global_load_lds(src + off + l * 16, (lds_void*)(smem + hb + off), 16, 0, 16 /* sc1 */);
    if (l < kChunkCols) {
      int pr;
      if constexpr (FUSED) {
        pr = lds_u16(lb + kGPairs + static_cast<uint32_t>((seq * kChunkCols + l) * 2));
        pr = pr == 0xffff ? -1 : pr;
      } else {
        pr = a.c_pairs[static_cast<int64_t>(ch) * kChunkCols + l];
      }
      lds_st4(lb + hb + a.hid_code_bytes + 4 * l, static_cast<uint32_t>(pr));
    }
    wait_vm<0>();
    lds_settle_all();
    if (l == 0) lds_st4(lb + kGReady, static_cast<uint32_t>(seq + 1));
  }
  // the call counters for the next call (every counter c, c + grid, ... below kMaxGrid,
  // so that all stay equal whatever grid the next call uses)
#pragma unroll 1
  for (int m = c + l * nwg; m < kMaxGrid; m += 64 * nwg) st_dev_u32(a.calls + m, call);
}

using ExpertsFn = void (*)(ExpArgs);

template <int R, bool DEC, bool TAG>
ExpertsFn pick_ns2(int ns2) {
  if (ns2 == 1) return experts_kernel<1, 1, R, DEC, TAG>;
  if (ns2 == 2) return experts_kernel<1, 2, R, DEC, TAG>;
  if (ns2 == 3) return experts_kernel<1, 3, R, DEC, TAG>;
  return experts_kernel<1, 4, R, DEC, TAG>;
}

// Kernel variants: form (grouped / decode, and the decode form's exchange) x NS2 =
// ceil(I/128) FC2 K steps x ring depth R (4, else what fits).
template <bool DEC, bool TAG>
ExpertsFn pick_kernel(int ns2, int R) {
  return R >= 4 ? pick_ns2<4, DEC, TAG>(ns2) : (R == 3 ? pick_ns2<3, DEC, TAG>(ns2) : pick_ns2<2, DEC, TAG>(ns2));
}

// LDS bytes of a variant (B, D: decode form's x plan).
template <int R, bool DEC>
size_t lds_ns2(int ns2, int g_cap, int u_cap, int IP, int B, int D) {
  if (ns2 == 1) return lds_bytes<1, R, 1, DEC>(g_cap, u_cap, IP, B, D);
  if (ns2 == 2) return lds_bytes<1, R, 2, DEC>(g_cap, u_cap, IP, B, D);
  if (ns2 == 3) return lds_bytes<1, R, 3, DEC>(g_cap, u_cap, IP, B, D);
  return lds_bytes<1, R, 4, DEC>(g_cap, u_cap, IP, B, D);
}
template <bool DEC>
size_t lds_for(int R, int ns2, int g_cap, int u_cap, int IP, int B, int D) {
  return R >= 4 ? lds_ns2<4, DEC>(ns2, g_cap, u_cap, IP, B, D)
                : (R == 3 ? lds_ns2<3, DEC>(ns2, g_cap, u_cap, IP, B, D) : lds_ns2<2, DEC>(ns2, g_cap, u_cap, IP, B, D));
}

// ------------------------------------------------------------------ host helpers
// The next-layer prefetch table of the options: rows <= kPfRows, each 16-byte aligned and
// below 2^31 bytes (a buffer resource's range), pieces counted in 32 bits.
bool pf_ok(const moe_run_opts_t& o) {
  if (o.ahead_rows < 0 || o.ahead_rows > kPfRows || (o.ahead_rows > 0 && o.ahead == nullptr)) return false;
  int64_t pieces = 0;
  for (int r = 0; r < o.ahead_rows; ++r) {
    const moe_prefetch_row_t& w = o.ahead[r];
    if (w.bytes >= (1ull << 31) || (w.bytes > 0 && (w.addr == nullptr || reinterpret_cast<uintptr_t>(w.addr) % 16)))
      return false;
    pieces += static_cast<int64_t>((w.bytes + 1023) / 1024);
  }
  return pieces < (1ll << 31);
}
void pf_table(const moe_run_opts_t& o, PfTable& t) {
  t.rows = 0;
  t.pieces = 0;
  for (int r = 0; r < o.ahead_rows; ++r) {
    t.row[r].addr = reinterpret_cast<uint64_t>(o.ahead[r].addr);
    t.row[r].bytes = static_cast<uint32_t>(o.ahead[r].bytes);
    t.row[r].first = static_cast<uint32_t>(t.pieces);
    t.pieces += static_cast<int>((o.ahead[r].bytes + 1023) / 1024);
    t.rows = r + 1;
  }
}

bool shape_ok(int64_t E, int64_t D, int64_t I) {
  return E >= 1 && E <= kMaxGroups && D >= 512 && D <= 16384 && D % 512 == 0 && I >= 32 && I <= 512 &&
         I % 32 == 0;
}

int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    cached[dev] = cus;
  }
  return cached[dev];
}

int device_lds_limit() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 65536;
  if (cached[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || v <= 0) v = 65536;
    cached[dev] = v;
  }
  return cached[dev];
}

// Allow the kernel variant its dynamic LDS (once per variant and size).
bool prepare_kernel(ExpertsFn fn, size_t lds) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                             static_cast<int>(lds)) == hipSuccess;
}

// Workgroups of one kernel variant that the device holds at once.
int resident_grid(ExpertsFn fn, size_t lds) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(fn), kWG, lds) !=
          hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  const int grid = per_cu * device_cus();
  return grid < kMaxGrid ? grid : kMaxGrid;
}

// The largest batch a workspace of ws_bytes serves (its layout is a function of it).
int ws_batch_capacity(int E, int D, int I, int K, size_t ws_bytes) {
  int lo = 0, hi = 65536 / K;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (ws_layout(E, D, I, K, mid).end <= ws_bytes) lo = mid; else hi = mid - 1;
  }
  return lo;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int launch_status() { return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP; }

int run_decode_whole(const moe_weights_t* wts, const moe_run_opts_t& o, const void* x, const int32_t* ids, int32_t B,
                     int32_t topk, void* ws, size_t ws_bytes, void* out, size_t out_bytes, void* stream);
bool whole_fits(const moe_weights_t* wts, int32_t B, int32_t topk);
bool grouped_fits(int E, int D, int I, int B, int K, int grid);
int run_grouped(const moe_weights_t* wts, const moe_run_opts_t& o, const void* plan, const void* units, const void* x,
                const int32_t* ids, int32_t B, int32_t topk, void* ws, size_t ws_bytes, void* out, void* stream);

// Checks, kernel variant, grid and arguments shared by both forms; enqueues one launch.
template <bool DEC>
int run_experts(const moe_weights_t* wts, const moe_run_opts_t* opts, const void* plan, const void* units,
                size_t units_bytes, const void* x, const int32_t* ids, int32_t B, int32_t topk, void* ws,
                size_t ws_bytes, void* out, size_t out_bytes, void* stream) {
  if (!wts || !ws || !out || B < 1 || topk < 1 || topk > 64 ||
      static_cast<int64_t>(B) * topk > 65535)  // pair indices are cached as u16, 0xffff = padding
    return MOE_EINVAL;
  const int E = wts->E, D = wts->D, I = wts->I;
  if (!shape_ok(E, D, I) || !wts->w13 || !wts->s13 || !wts->w2 || !wts->s2) return MOE_EINVAL;
  moe_run_opts_t o;
  std::memset(&o, 0, sizeof(o));
  if (opts) o = *opts;
  if (o.hidden_rule < 0 || o.hidden_rule > 2 || o.grid < 0 || o.col_tiles < 0 || o.col_tiles > (DEC ? 1 : 2) ||
      (o.ring != 0 && (o.ring < 2 || o.ring > 4)) || o.fc2_claims < 0 || o.fc2_claims > 1 || !pf_ok(o) ||
      ((o.hidden_codes_dev == nullptr) != (o.hidden_scales_dev == nullptr)))
    return MOE_EINVAL;
  if (!DEC && (o.plan_dev != nullptr || o.status_dev != nullptr || o.exchange != 0 || o.ahead_rows != 0))
    return MOE_EINVAL;  // decode-form options
  if (o.exchange < 0 || o.exchange > (DEC ? 2 : 0)) return MOE_EINVAL;
  if (out_bytes < static_cast<size_t>(B) * topk * D * 2) return MOE_ENOSPACE;
  if (!DEC && units_bytes < units_layout(B, topk, E).end) return MOE_ENOSPACE;
  if (DEC && o.plan_bytes != 0 && o.plan_dev == nullptr) return MOE_EINVAL;
  if (DEC && o.plan_dev != nullptr && o.plan_bytes < static_cast<size_t>(B) * D / 32 * 33) return MOE_ENOSPACE;
  // the decode form's default exchange: whole-K blocks where the batch fits its limits,
  // else finished split blocks
  if (DEC && o.exchange == 0 && whole_fits(wts, B, topk))
    return run_decode_whole(wts, o, x, ids, B, topk, ws, ws_bytes, out, out_bytes, stream);
  if (o.ahead_rows != 0 || o.fc2_claims != 0) return MOE_EINVAL;  // options of the whole-K kernel only
  // the grouped form's default: whole-K FC1 blocks over 32-column chunks (col_tiles 0 or 2)
  // where the batch fits its tables; col_tiles 1 asks for the split-block kernel
  if (!DEC && o.col_tiles != 1 && grouped_fits(E, D, I, B, topk, o.grid ? o.grid : device_cus()))
    return run_grouped(wts, o, plan, units, nullptr, nullptr, B, topk, ws, ws_bytes, out, stream);
  if (!DEC && o.col_tiles == 2) return MOE_EINVAL;
  const int B_cap = ws_batch_capacity(E, D, I, topk, ws_bytes);
  if (B_cap < B) return MOE_ENOSPACE;
  const WsLayout L = ws_layout(E, D, I, topk, B_cap);
  const int64_t U = static_cast<int64_t>(B) * topk;
  const int g_cap = static_cast<int>(U < E ? U : E);
  const int64_t u_bound = g_cap + (U + 7) / 8;
  const int u_cap = DEC ? g_cap : static_cast<int>(U < u_bound ? U : u_bound);
  const int IP = (I + 127) / 128 * 128, ns2 = IP / 128;
  // the deepest ring that fits next to the unit table (and the decode form's x plan)
  int R = o.ring ? o.ring : 4;
  if (!o.ring)
    while (R > 2 && lds_for<DEC>(R, ns2, g_cap, u_cap, IP, B, D) > static_cast<size_t>(device_lds_limit())) --R;
  const size_t lds = lds_for<DEC>(R, ns2, g_cap, u_cap, IP, B, D);
  if (lds > static_cast<size_t>(device_lds_limit())) return MOE_EINVAL;  // unit table too large for LDS
  const bool tag = DEC && o.exchange == 1;
  const ExpertsFn fn = tag ? pick_kernel<DEC, DEC>(ns2, R) : pick_kernel<DEC, false>(ns2, R);
  if (!prepare_kernel(fn, lds)) return MOE_EHIP;
  const int cap = resident_grid(fn, lds);
  if (o.grid > cap) return MOE_EINVAL;  // the grid must be co-resident
  const int grid = o.grid ? o.grid : cap;

  uint8_t* base = static_cast<uint8_t*>(ws);
  ExpArgs a;
  std::memset(&a, 0, sizeof(a));
  a.w13p = static_cast<const uint8_t*>(wts->w13);
  a.s13p = static_cast<const uint8_t*>(wts->s13);
  a.w2p = static_cast<const uint8_t*>(wts->w2);
  a.s2p = static_cast<const uint8_t*>(wts->s2);
  if (DEC) {
    a.x = static_cast<const uint16_t*>(x);
    a.ids = ids;
    a.plan_dump = static_cast<uint8_t*>(o.plan_dev);
    a.err = o.status_dev ? static_cast<int32_t*>(o.status_dev) : reinterpret_cast<int32_t*>(base + L.status);
    a.dpart = reinterpret_cast<uint64_t*>(base + L.partials);
  } else {
    a.xcodes = static_cast<const uint8_t*>(plan);
    a.xscales = a.xcodes + static_cast<int64_t>(B) * D;
    a.plan_bytes = static_cast<uint32_t>(static_cast<int64_t>(B) * D / 32 * 33);
    a.tbl = table_at(static_cast<uint8_t*>(const_cast<void*>(units)), units_layout(B, topk, E));
    a.err = a.tbl.hdr + 3;
  }
  a.calls = reinterpret_cast<uint32_t*>(base + L.calls);
  a.arrive = reinterpret_cast<uint32_t*>(base + L.arrive);
  a.flags = reinterpret_cast<uint32_t*>(base + L.flags);
  a.hcodes = base + L.hcodes;
  a.hscales = base + L.hscales;
  a.partials = reinterpret_cast<float*>(base + L.partials);
  a.out = static_cast<uint16_t*>(out);
  a.dump_codes = static_cast<uint8_t*>(o.hidden_codes_dev);
  a.dump_scales = static_cast<uint8_t*>(o.hidden_scales_dev);
  a.D = D;
  a.I = I;
  a.HB = I / 32;
  a.NS1 = D / 128;
  a.NSP = a.NS1 / 2;
  a.U2 = D / 16 / (ns2 == 1 ? 8 : (ns2 == 2 ? 4 : 2));
  a.IP = IP;
  a.g_cap = g_cap;
  a.u_cap = u_cap;
  a.K = topk;
  a.B = B;
  a.E = E;
  a.qmin = tag ? (a.NSP + 2) / 3 : 0;
  a.floor_rule = o.hidden_rule == 2 || (o.hidden_rule == 0 && I == 384);
  hipLaunchKernelGGL(fn, dim3(grid), dim3(kWG), lds, as_stream(stream), a);
  return launch_status();
}


// ------------------------------------------------- grouped form, whole-K FC1 blocks (host)
using GFn = void (*)(GArgs);
GFn pick_g(int ns2, bool fused) {
  switch (ns2) {
    case 1: return fused ? grouped_kernel<1, true> : grouped_kernel<1, false>;
    case 2: return fused ? grouped_kernel<2, true> : grouped_kernel<2, false>;
    default: return fused ? grouped_kernel<3, true> : grouped_kernel<3, false>;
  }
}

// LDS layout of the grouped kernel for (D, I).
struct GLds {
  uint32_t colb, code_bytes, hid_bytes;   // hidden column bytes; the hidden buffer's codes, and all of it
  uint32_t o_ring, o_hid;
  size_t total;
};
GLds grouped_lds(int D, int I) {
  (void)D;
  GLds g;
  const int IP = (I + 127) / 128 * 128;
  g.colb = static_cast<uint32_t>(IP + 16);
  g.code_bytes = (kChunkCols * g.colb + 1023u) / 1024u * 1024u;
  g.hid_bytes = g.code_bytes + 4u * kChunkCols;
  g.o_ring = (kGTables + 15u) / 16u * 16u;
  g.o_hid = g.o_ring + kGStream * kGR * kGSlot;  // FC1's staging areas, then FC2's hidden buffer
  const uint32_t stage = kGStream * kGStage;
  g.total = g.o_hid + (g.hid_bytes > stage ? g.hid_bytes : stage);
  return g;
}
constexpr size_t kGLdsMax = 160 * 1024;  // LDS of a gfx950 workgroup

// The grouped kernel's limits: its LDS tables hold kGChunks chunks and kGItems FC1 items
// per workgroup; I <= 384 (three FC2 K steps: nine waves share a SIMD's registers, and
// a fourth K step would not fit them); its LDS layout fits.
bool grouped_fits(int E, int D, int I, int B, int K, int grid) {
  const int64_t U = static_cast<int64_t>(B) * K;
  const int64_t chunks = max_chunks_for(U, U < E ? U : E);
  const int64_t items = (chunks * (I / 32) + grid - 1) / grid;
  return I <= 384 && chunks <= kGChunks && items <= kGItems && grouped_lds(D, I).total <= kGLdsMax;
}
// The one-launch form also keeps the pairs of a workgroup's FC2 chunks (at most kGSeqMax)
// and builds the chunk table in the ring's LDS (token bitmasks [B/32][E], two counts per
// expert, a row index per chunk and the rows of the needed chunks) before any DMA; pair
// indices are u16.
bool grouped_fused_fits(int E, int D, int I, int B, int K, int grid) {
  const int64_t U = static_cast<int64_t>(B) * K;
  const int64_t chunks = max_chunks_for(U, U < E ? U : E);
  const int64_t TPE = D / 16, cap = (chunks * TPE + grid - 1) / grid;
  const int64_t seqs = (cap + TPE - 1) / TPE + 1;
  const int64_t scratch = (static_cast<int64_t>((B + 31) / 32) * E + 2 * E + kGChunks) * 4 +
                          (kGItems + kGSeqMax) * (2 * kChunkCols + 4);
  return grouped_fits(E, D, I, B, K, grid) && seqs <= kGSeqMax && U < 0xffff && E <= 2 * kGWG &&
         scratch <= static_cast<int64_t>(kGStream) * kGR * kGSlot;
}

// The grouped kernel.  units != NULL: on the plan and unit table of moe_plan_group;
// units == NULL: the one-launch form, which makes them itself from x and ids.
int run_grouped(const moe_weights_t* wts, const moe_run_opts_t& o, const void* plan, const void* units, const void* x,
                const int32_t* ids, int32_t B, int32_t topk, void* ws, size_t ws_bytes, void* out, void* stream) {
  const bool fused = units == nullptr;
  const int E = wts->E, D = wts->D, I = wts->I;
  const int IP = (I + 127) / 128 * 128, ns2 = IP / 128, HB = I / 32, NS1 = D / 128;
  const int B_cap = ws_batch_capacity(E, D, I, topk, ws_bytes);
  if (B_cap < B) return MOE_ENOSPACE;
  const WsLayout L = ws_layout(E, D, I, topk, B_cap);
  const UnitsLayout UL = units_layout(B, topk, E);
  const GLds G = grouped_lds(D, I);
  const size_t lds = G.total;
  if (lds > static_cast<size_t>(device_lds_limit())) return MOE_EINVAL;
  const GFn fn = pick_g(ns2, fused);
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                          static_cast<int>(lds)) != hipSuccess)
    return MOE_EHIP;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(fn), kGWG, lds) !=
          hipSuccess || per_cu < 1)
    per_cu = 1;
  int cap = per_cu * device_cus();
  if (cap > kMaxGrid) cap = kMaxGrid;
  if (o.grid > cap) return MOE_EINVAL;  // the grid must be co-resident
  const int grid = o.grid ? o.grid : cap;
  if (!(fused ? grouped_fused_fits(E, D, I, B, topk, grid) : grouped_fits(E, D, I, B, topk, grid))) return MOE_EINVAL;

  uint8_t* base = static_cast<uint8_t*>(ws);
  uint8_t* ub = static_cast<uint8_t*>(const_cast<void*>(units));
  GArgs a;
  std::memset(&a, 0, sizeof(a));
  a.w13p = static_cast<const uint8_t*>(wts->w13);
  a.s13p = static_cast<const uint8_t*>(wts->s13);
  a.w2p = static_cast<const uint8_t*>(wts->w2);
  a.s2p = static_cast<const uint8_t*>(wts->s2);
  a.plan = static_cast<const uint8_t*>(plan);
  if (fused) {
    // the plan goes to the caller's plan buffer when there is one, else to the workspace
    a.plan = o.plan_dev != nullptr ? static_cast<const uint8_t*>(o.plan_dev) : base + L.gplan;
    a.x = static_cast<const uint8_t*>(x);
    a.ids = ids;
    a.pflags = reinterpret_cast<uint32_t*>(base + L.gpflags);
    a.E = E;
  } else {
    a.hdr = reinterpret_cast<const int32_t*>(ub + UL.hdr);
    a.c_expert = reinterpret_cast<const int32_t*>(ub + UL.c_expert);
    a.c_cols = reinterpret_cast<const int32_t*>(ub + UL.c_cols);
    a.c_pairs = reinterpret_cast<const int32_t*>(ub + UL.c_pairs);
  }
  a.out = static_cast<uint16_t*>(out);
  a.hid = base + L.ghid;
  a.flags = reinterpret_cast<uint32_t*>(base + L.gflags);
  a.calls = reinterpret_cast<uint32_t*>(base + L.gcalls);
  a.err = fused ? (o.status_dev ? static_cast<int32_t*>(o.status_dev) : reinterpret_cast<int32_t*>(base + L.status))
                : reinterpret_cast<int32_t*>(ub + UL.hdr) + 3;
  a.dump_codes = static_cast<uint8_t*>(o.hidden_codes_dev);
  a.dump_scales = static_cast<uint8_t*>(o.hidden_scales_dev);
  a.B = B;
  a.K = topk;
  a.kinv = (uint64_t{1} << 32) / static_cast<uint64_t>(topk) + 1u;
  a.D = D;
  a.I = I;
  a.HB = HB;
  a.NS1 = NS1;
  a.IP = IP;
  a.floor_rule = o.hidden_rule == 2 || (o.hidden_rule == 0 && I == 384);
  a.max_chunks = static_cast<int>(UL.max_chunks);
  a.plan_bytes = static_cast<uint32_t>(static_cast<int64_t>(B) * D / 32 * 33);
  a.out_bytes = static_cast<uint32_t>(static_cast<int64_t>(B) * topk * D * 2);
  a.colb = G.colb;
  a.o_ring = G.o_ring;
  a.o_hid = G.o_hid;
  a.hid_code_bytes = G.code_bytes;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(kGWG), lds, as_stream(stream), a);
  return launch_status();
}

// The whole step of a batch of B > 8 in one launch: the grouped kernel making its plan and
// chunk table itself (the options of the grouped form; plan_dev and status_dev as in the
// decode form).
int run_step_grouped(const moe_weights_t* wts, const moe_run_opts_t* opts, const void* x, const int32_t* ids,
                     int32_t B, int32_t topk, void* ws, size_t ws_bytes, void* out, size_t out_bytes, void* stream) {
  if (!wts || !ws || !out || B < 1 || topk < 1 || topk > 64 || static_cast<int64_t>(B) * topk >= 0xffff)
    return MOE_EINVAL;
  const int E = wts->E, D = wts->D, I = wts->I;
  if (!shape_ok(E, D, I) || !wts->w13 || !wts->s13 || !wts->w2 || !wts->s2) return MOE_EINVAL;
  moe_run_opts_t o;
  std::memset(&o, 0, sizeof(o));
  if (opts) o = *opts;
  if (o.hidden_rule < 0 || o.hidden_rule > 2 || o.grid < 0 || (o.col_tiles != 0 && o.col_tiles != 2) ||
      (o.ring != 0 && (o.ring < 2 || o.ring > 4)) || o.exchange != 0 || o.fc2_claims != 0 || o.ahead_rows != 0 ||
      ((o.hidden_codes_dev == nullptr) != (o.hidden_scales_dev == nullptr)) ||
      (o.plan_bytes != 0 && o.plan_dev == nullptr))
    return MOE_EINVAL;
  if (out_bytes < static_cast<size_t>(B) * topk * D * 2) return MOE_ENOSPACE;
  if (o.plan_dev != nullptr && o.plan_bytes < static_cast<size_t>(B) * D / 32 * 33) return MOE_ENOSPACE;
  if (!grouped_fused_fits(E, D, I, B, topk, o.grid ? o.grid : device_cus())) return MOE_EINVAL;
  return run_grouped(wts, o, nullptr, nullptr, x, ids, B, topk, ws, ws_bytes, out, stream);
}

// ------------------------------------------------- decode form, whole-K FC1 blocks (host)
using QFn = void (*)(QArgs);
// wide: an expert's hidden can exceed 512 pairs (more than four tokens at I = 384), so
// the loader polls it in one pass (two slots per wave only)
// claims: a separate instantiation (two slots per wave only), so that the static form
// keeps its own code
template <int NS2>
QFn pick_q_r(int R, bool wide, bool claims) {
  if (claims) return wide ? decode_whole_kernel<NS2, 2, true, true> : decode_whole_kernel<NS2, 2, false, true>;
  switch (R) {
    case 2: return wide ? decode_whole_kernel<NS2, 2, true, false> : decode_whole_kernel<NS2, 2, false, false>;
    case 3: return decode_whole_kernel<NS2, 3, false, false>;
    default: return decode_whole_kernel<NS2, 4, false, false>;
  }
}
QFn pick_q(int ns2, int R, bool wide, bool claims) {
  switch (ns2) {
    case 1: return pick_q_r<1>(R, wide, claims);
    case 2: return pick_q_r<2>(R, wide, claims);
    case 3: return pick_q_r<3>(R, wide, claims);
    default: return pick_q_r<4>(R, wide, claims);
  }
}

struct QLds {
  uint32_t o_red, o_hid, o_xq, o_xs, o_ring, xstr, xsstr, hid_bytes, red_wave;
  int cb;
  size_t bytes(int R) const { return o_ring + static_cast<size_t>(kQStream) * R * kQSlot; }
};
QLds q_lds(int B, int D, int IP) {
  QLds m;
  auto a16 = [](uint32_t v) { return (v + 15u) & ~15u; };
  m.cb = B < 8 ? B : 8;  // token columns of a group
  m.red_wave = 256u * static_cast<uint32_t>(m.cb);
  m.o_red = a16(kQTables);
  m.hid_bytes = static_cast<uint32_t>(m.cb) * (static_cast<uint32_t>(IP) + kQHB);
  m.o_hid = m.o_red + kQStream * m.red_wave;
  m.xstr = static_cast<uint32_t>(D) + 16u;
  m.xsstr = static_cast<uint32_t>(D) / 32u;
  m.o_xq = a16(m.o_hid + 2u * m.hid_bytes);
  m.o_xs = a16(m.o_xq + static_cast<uint32_t>(B) * m.xstr);
  m.o_ring = a16(m.o_xs + static_cast<uint32_t>(B) * m.xsstr);
  return m;
}

// The limits of the decode form with whole-K FC1 blocks: at most 128 distinct experts,
// B*topk <= 576 routes, B*D/32 <= 4 * 576 blocks of x, I <= 512.
bool whole_fits(const moe_weights_t* wts, int32_t B, int32_t topk) {
  const int64_t routes = static_cast<int64_t>(B) * topk;
  const int64_t gmax = routes < wts->E ? routes : wts->E;
  return wts->I <= 512 && gmax <= kQGMax && routes <= kQWG &&
         static_cast<int64_t>(B) * wts->D / 32 <= static_cast<int64_t>(kQXBlk) * kQWG;
}

// The decode form with whole-K FC1 blocks on the given workspace areas: the call
// counters [kMaxGrid], the FC2 claim counters [kMaxGrid], the default status word and
// the hidden exchange [kQGMax][8][IP/4 + kQHB] pairs (from a caller's workspace, or from
// the allocation-free entry point's fixed scratch).
int launch_decode_whole(const moe_weights_t* wts, const moe_run_opts_t& o, const void* x, const int32_t* ids,
                        int32_t B, int32_t topk, uint32_t* calls, uint64_t* claims, int32_t* status, uint64_t* hq,
                        void* out, void* stream);

// The decode form with whole-K FC1 blocks (moe_run_opts_t.exchange == 0, the default,
// for batches within whole_fits).
int run_decode_whole(const moe_weights_t* wts, const moe_run_opts_t& o, const void* x, const int32_t* ids, int32_t B,
                     int32_t topk, void* ws, size_t ws_bytes, void* out, size_t out_bytes, void* stream) {
  const int E = wts->E, D = wts->D, I = wts->I;
  if (!whole_fits(wts, B, topk)) return MOE_EINVAL;
  const int B_cap = ws_batch_capacity(E, D, I, topk, ws_bytes);
  if (B_cap < B) return MOE_ENOSPACE;
  const WsLayout L = ws_layout(E, D, I, topk, B_cap);
  (void)out_bytes;
  uint8_t* base = static_cast<uint8_t*>(ws);
  return launch_decode_whole(wts, o, x, ids, B, topk, reinterpret_cast<uint32_t*>(base + L.qcalls),
                             reinterpret_cast<uint64_t*>(base + L.qclaims), reinterpret_cast<int32_t*>(base + L.status),
                             reinterpret_cast<uint64_t*>(base + L.qhq), out, stream);
}

int launch_decode_whole(const moe_weights_t* wts, const moe_run_opts_t& o, const void* x, const int32_t* ids,
                        int32_t B, int32_t topk, uint32_t* calls, uint64_t* claims, int32_t* status, uint64_t* hq,
                        void* out, void* stream) {
  const int E = wts->E, D = wts->D, I = wts->I;
  const int IP = (I + 127) / 128 * 128, ns2 = IP / 128;
  const QLds m = q_lds(B, D, IP);
  const size_t limit = static_cast<size_t>(device_lds_limit());
  // two slots per wave by default: measured fastest at the decode sizes (B = 1: 13.9 us
  // with two, 14.5 with three, 15.0 with four; B = 8: 35.7, 37.4, -).  More requests in
  // flight only lengthen each one's latency, and a deeper ring brings FC2 prefetch
  // forward into FC1's critical stream.
  int R = 2;
  if (o.ring) R = o.ring < 2 ? 2 : (o.ring > 4 ? 4 : o.ring);
  while (R > 2 && m.bytes(R) > limit) --R;
  if (m.bytes(R) > limit) return MOE_EINVAL;
  const size_t lds = m.bytes(R);
  if (o.fc2_claims && R != 2) return MOE_EINVAL;  // claims run with two slots per wave
  const QFn fn = pick_q(ns2, R, m.cb * (I / 4 + I / 32) > 8 * 64, o.fc2_claims != 0);
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                          static_cast<int>(lds)) != hipSuccess)
    return MOE_EHIP;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(fn), kQWG, lds) !=
          hipSuccess || per_cu < 1)
    per_cu = 1;
  int cap = per_cu * device_cus();
  if (cap > kMaxGrid) cap = kMaxGrid;
  if (o.grid > cap) return MOE_EINVAL;  // the grid must be co-resident
  const int grid = o.grid ? o.grid : cap;

  QArgs a;
  std::memset(&a, 0, sizeof(a));
  a.w13p = static_cast<const uint8_t*>(wts->w13);
  a.s13p = static_cast<const uint8_t*>(wts->s13);
  a.w2p = static_cast<const uint8_t*>(wts->w2);
  a.s2p = static_cast<const uint8_t*>(wts->s2);
  a.x = static_cast<const uint16_t*>(x);
  a.ids = ids;
  a.out = static_cast<uint16_t*>(out);
  a.hq = hq;
  a.hq_words = IP / 4 + kQHB;
  a.calls = calls;
  a.claims = claims;
  a.zone = o.fc2_claims ? kQZone : 0;
  a.err = o.status_dev ? static_cast<int32_t*>(o.status_dev) : status;
  a.dump_codes = static_cast<uint8_t*>(o.hidden_codes_dev);
  a.dump_scales = static_cast<uint8_t*>(o.hidden_scales_dev);
  a.plan_dump = static_cast<uint8_t*>(o.plan_dev);
  a.B = B;
  a.K = topk;
  a.E = E;
  a.D = D;
  a.I = I;
  a.HB = I / 32;
  a.NS1 = D / 128;
  a.IP = IP;
  a.floor_rule = o.hidden_rule == 2 || (o.hidden_rule == 0 && I == 384);
  a.o_red = m.o_red;
  a.o_hid = m.o_hid;
  a.o_xq = m.o_xq;
  a.o_xs = m.o_xs;
  a.o_ring = m.o_ring;
  a.xstr = m.xstr;
  a.xsstr = m.xsstr;
  a.hid_bytes = m.hid_bytes;
  a.cb = m.cb;
  a.red_wave = m.red_wave;
  pf_table(o, a.pf);
  hipLaunchKernelGGL(fn, dim3(grid), dim3(kQWG), lds, as_stream(stream), a);
  return launch_status();
}

// ------------------------------------------- the allocation-free entry point's scratch
// moe_decode_run_noalloc keeps what moe_decode_run keeps in the caller's workspace --
// the call counters, the status word and the call-tagged hidden exchange -- in this
// file-scope array instead: one copy per device, zero when the code object is loaded,
// kept until the process ends.  Every quantity in it is tagged with call numbers, so
// no call clears anything.  Host code never uses the array's name as an address: the
// device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchCalls = 0;                                  // u32 [kMaxGrid]
constexpr size_t kScratchStatus = kScratchCalls + kMaxGrid * 4;      // i32 status word
constexpr size_t kScratchClaims = kScratchStatus + 256;              // u64 [kMaxGrid] FC2 claim counters
constexpr size_t kScratchHq = kScratchClaims + kMaxGrid * 8;         // u64 [kQGMax][8][512 / 4 + kQHB]
constexpr size_t kScratchBytes = kScratchHq + static_cast<size_t>(kQGMax) * 8 * (512 / 4 + kQHB) * 8;
static_assert(kScratchClaims % 256 == 0 && kScratchHq % 256 == 0, "aligned areas");
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

// The device address of this device's copy of `scratch` (nullptr if it cannot be had).
uint8_t* scratch_ptr() {
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    ptrs[dev] = p;
  }
  return static_cast<uint8_t*>(ptrs[dev]);
}
}  // namespace

// ====================================================================== C ABI
extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument or unsupported shape";
    case MOE_ENOSPACE: return "buffer too small";
    case MOE_EHIP: return "HIP launch or runtime error";
    case MOE_ELIMIT: return "batch beyond the fixed scratch of the allocation-free entry point";
    default: return "unknown status";
  }
}

size_t moe_plan_bytes(int32_t B, int32_t D) {
  if (B < 1 || D < 32 || D % 32) return 0;
  return static_cast<size_t>(B) * D + static_cast<size_t>(B) * (D / 32);
}

size_t moe_units_bytes(int32_t B, int32_t topk, int32_t E) {
  if (B < 1 || topk < 1 || topk > 64 || E < 1 || E > kMaxGroups || static_cast<int64_t>(B) * topk > 65536) return 0;
  return units_layout(B, topk, E).end;
}

size_t moe_workspace_bytes(int32_t E, int32_t D, int32_t I, int32_t B_max, int32_t topk) {
  if (!shape_ok(E, D, I) || B_max < 1 || topk < 1 || topk > 64 || static_cast<int64_t>(B_max) * topk > 65536)
    return 0;
  return ws_layout(E, D, I, topk, B_max).end;
}

int moe_work_split(int32_t form, int32_t groups, int32_t D, int32_t I, int32_t grid, int32_t claims_ring,
                   int32_t* split, int32_t* items) {
  if ((form != 0 && form != 1) || groups < 0 || !shape_ok(1, D, I) || grid < 1 || grid > kMaxGrid ||
      split == nullptr || claims_ring < 0 || claims_ring == 1 || claims_ring > 4 || (form == 1 && claims_ring != 0))
    return MOE_EINVAL;
  const int HB = I / 32, NS1 = D / 128, NS2 = (I + 127) / 128;
  if (form == 0 && (groups > kQGMax || HB > kQHB)) return MOE_EINVAL;
  if (form == 1 && groups > kGChunks) return MOE_EINVAL;
  for (int c = 0; c < grid; ++c) {
    const QWork q = form == 0 ? q_work(groups, HB, NS1, D, grid, c, 0, q_item_tiles(D, NS2))
                              : g_work(groups, HB, NS1, D, grid, c);
    int zb = q.first2 + q.n2;
    const int Z = claims_ring ? q_zone(q, kQZone, claims_ring, zb) : 0;
    int32_t* r = split + 6 * c;
    r[0] = q.n1;
    r[1] = q.first2;
    r[2] = q.n2;
    r[3] = form == 0 ? kQStream : kGStream;
    r[4] = zb;
    r[5] = Z;
  }
  if (items != nullptr) {
    for (int i = 0; i < groups * HB; ++i) {
      int g = i / HB, j = i - (i / HB) * HB;
      if (form == 1) g_item(i, groups, HB, g, j);
      items[2 * i] = g;
      items[2 * i + 1] = j;
    }
  }
  return MOE_OK;
}

int moe_grouped_runs(int32_t chunks, const int32_t* chunk_cols, int32_t D, int32_t I, int32_t grid, int32_t* runs) {
  if (chunks < 0 || chunks > kGChunks || !shape_ok(1, D, I) || I > 384 || grid < 1 || grid > kMaxGrid ||
      runs == nullptr || (chunks > 0 && chunk_cols == nullptr))
    return MOE_EINVAL;
  int64_t cols = 0;
  for (int ch = 0; ch < chunks; ++ch) {
    if (chunk_cols[ch] < 1 || chunk_cols[ch] > kChunkCols) return MOE_EINVAL;
    cols += chunk_cols[ch];
  }
  if (cols > 65536) return MOE_EINVAL;
  for (int c = 0; c < grid; ++c) g_run_host(chunk_cols, chunks, D, I, grid, c, runs[2 * c], runs[2 * c + 1]);
  return MOE_OK;
}

int moe_packed_weight_bytes(int32_t E, int32_t D, int32_t I, size_t* w13_bytes, size_t* s13_bytes,
                            size_t* w2_bytes, size_t* s2_bytes) {
  if (!shape_ok(E, D, I)) return MOE_EINVAL;
  const size_t NS2 = (I + 127) / 128, NQ2 = (NS2 + 3) / 4;
  if (w13_bytes) *w13_bytes = static_cast<size_t>(E) * 2 * I * (D / 2);
  if (s13_bytes) *s13_bytes = static_cast<size_t>(E) * 2 * I * (D / 32);
  if (w2_bytes) *w2_bytes = static_cast<size_t>(E) * (D / 16) * NS2 * 1024;
  if (s2_bytes) *s2_bytes = static_cast<size_t>(E) * (D / 16) * NQ2 * 256;
  return MOE_OK;
}

int moe_pack_weights(int32_t E, int32_t D, int32_t I, const void* w13, const void* s13, const void* w2,
                     const void* s2, void* w13p, void* s13p, void* w2p, void* s2p, void* stream) {
  if (!shape_ok(E, D, I) || !w13 || !s13 || !w2 || !s2 || !w13p || !s13p || !w2p || !s2p) return MOE_EINVAL;
  hipStream_t st = as_stream(stream);
  const int HB = I / 32, NS1 = D / 128, NS2 = (I + 127) / 128, NQ2 = (NS2 + 3) / 4;
  auto blocks = [](int64_t n) { return static_cast<unsigned>((n + 255) / 256); };
  const int64_t n1 = static_cast<int64_t>(E) * HB * NS1 * 256, n2 = static_cast<int64_t>(E) * HB * NS1 * 64;
  const int64_t n3 = static_cast<int64_t>(E) * (D / 16) * NS2 * 64, n4 = static_cast<int64_t>(E) * (D / 16) * NQ2 * 64;
  hipLaunchKernelGGL(pack_w13_codes, dim3(blocks(n1)), dim3(256), 0, st, static_cast<const uint4*>(w13),
                     static_cast<uint4*>(w13p), E, D, I);
  hipLaunchKernelGGL(pack_w13_scales, dim3(blocks(n2)), dim3(256), 0, st, static_cast<const uint8_t*>(s13),
                     static_cast<uint32_t*>(s13p), E, D, I);
  hipLaunchKernelGGL(pack_w2_codes, dim3(blocks(n3)), dim3(256), 0, st, static_cast<const uint4*>(w2),
                     static_cast<uint4*>(w2p), E, D, I);
  hipLaunchKernelGGL(pack_w2_scales, dim3(blocks(n4)), dim3(256), 0, st, static_cast<const uint8_t*>(s2),
                     static_cast<uint32_t*>(s2p), E, D, I);
  return launch_status();
}

int moe_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws || ws_bytes < 256) return MOE_EINVAL;
  return hipMemsetAsync(ws, 0, ws_bytes, as_stream(stream)) == hipSuccess ? MOE_OK : MOE_EHIP;
}

int moe_plan(const void* x, int32_t B, int32_t D, void* plan, size_t plan_bytes, void* stream) {
  if (!x || !plan || B < 1 || D < 32 || D % 32) return MOE_EINVAL;
  if (plan_bytes < moe_plan_bytes(B, D)) return MOE_ENOSPACE;
  const int64_t nblocks = static_cast<int64_t>(B) * (D / 32);
  uint8_t* codes = static_cast<uint8_t*>(plan);
  hipLaunchKernelGGL(plan_kernel, dim3(static_cast<unsigned>((4 * nblocks + 255) / 256)), dim3(256), 0,
                     as_stream(stream), static_cast<const uint8_t*>(x), nblocks, codes,
                     codes + static_cast<int64_t>(B) * D);
  return launch_status();
}

int moe_combine(const void* rows, size_t rows_bytes, const float* weights, int32_t B, int32_t topk, int32_t D,
                void* out, size_t out_bytes, void* stream) {
  if (!rows || !weights || !out || B < 1 || topk < 1 || D < 8 || D % 8) return MOE_EINVAL;
  if (rows_bytes < static_cast<size_t>(B) * topk * D * 2 || out_bytes < static_cast<size_t>(B) * D * 2)
    return MOE_ENOSPACE;
  const int64_t n = static_cast<int64_t>(B) * (D / 8);
  hipLaunchKernelGGL(combine_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, as_stream(stream),
                     static_cast<const uint16_t*>(rows), weights, B, topk, D, static_cast<uint16_t*>(out));
  return launch_status();
}

int moe_group(const int32_t* ids, int32_t B, int32_t topk, int32_t E, void* units, size_t units_bytes,
              void* stream) {
  if (!ids || !units || B < 1 || topk < 1 || topk > 64 || E < 1 || E > kMaxGroups ||
      static_cast<int64_t>(B) * topk > 65536)
    return MOE_EINVAL;
  const int W = (B + 31) / 32;
  const size_t lds = group_lds_words(B, topk, E) * 4;
  if (lds > 60 * 1024) return MOE_EINVAL;
  const UnitsLayout L = units_layout(B, topk, E);
  if (units_bytes < L.end) return MOE_ENOSPACE;
  const Table t = table_at(static_cast<uint8_t*>(units), L);
  hipLaunchKernelGGL(group_kernel, dim3(kGroupParts), dim3(kGroupThreads), lds, as_stream(stream), ids, B, topk, E,
                     W, t);
  return launch_status();
}

int moe_plan_group(const void* x, const int32_t* ids, int32_t B, int32_t D, int32_t topk, int32_t E, void* plan,
                   size_t plan_bytes, void* units, size_t units_bytes, void* stream) {
  if (!x || !plan || !ids || !units || B < 1 || D < 32 || D % 32 || topk < 1 || topk > 64 || E < 1 ||
      E > kMaxGroups || static_cast<int64_t>(B) * topk > 65536)
    return MOE_EINVAL;
  if (plan_bytes < moe_plan_bytes(B, D)) return MOE_ENOSPACE;
  const int W = (B + 31) / 32;
  const size_t lds = group_lds_words(B, topk, E) * 4;
  if (lds > 60 * 1024) return MOE_EINVAL;
  const UnitsLayout L = units_layout(B, topk, E);
  if (units_bytes < L.end) return MOE_ENOSPACE;
  const Table t = table_at(static_cast<uint8_t*>(units), L);
  const int64_t nblocks = static_cast<int64_t>(B) * (D / 32);
  uint8_t* codes = static_cast<uint8_t*>(plan);
  const unsigned grid = kGroupParts + static_cast<unsigned>((4 * nblocks + kGroupThreads - 1) / kGroupThreads);
  hipLaunchKernelGGL(plan_group_kernel, dim3(grid), dim3(kGroupThreads), lds, as_stream(stream),
                     static_cast<const uint8_t*>(x), nblocks, codes, codes + static_cast<int64_t>(B) * D, ids, B,
                     topk, E, W, t);
  return launch_status();
}

int moe_units_export(const void* units, size_t units_bytes, int32_t B, int32_t topk, int32_t E, void* header,
                     void* unit_expert, void* unit_rows, int32_t max_units, void* stream) {
  if (!units || !header || !unit_expert || !unit_rows || B < 1 || topk < 1 || E < 1 || max_units < 0)
    return MOE_EINVAL;
  const UnitsLayout L = units_layout(B, topk, E);
  if (units_bytes < L.end) return MOE_ENOSPACE;
  const int64_t U = static_cast<int64_t>(B) * topk;
  const int64_t n = max_units < U ? max_units : U;
  const uint8_t* base = static_cast<const uint8_t*>(units);
  hipStream_t st = as_stream(stream);
  if (hipMemcpyAsync(header, base + L.hdr, 16, hipMemcpyDeviceToDevice, st) != hipSuccess) return MOE_EHIP;
  if (n > 0) {
    if (hipMemcpyAsync(unit_expert, base + L.unit_expert, n * 4, hipMemcpyDeviceToDevice, st) != hipSuccess)
      return MOE_EHIP;
    if (hipMemcpyAsync(unit_rows, base + L.unit_rows, n * 32, hipMemcpyDeviceToDevice, st) != hipSuccess)
      return MOE_EHIP;
  }
  return MOE_OK;
}

int moe_experts_run(const moe_weights_t* wts, const moe_run_opts_t* opts, const void* plan, const void* units,
                    size_t units_bytes, int32_t B, int32_t topk, void* ws, size_t ws_bytes, void* out,
                    size_t out_bytes, void* stream) {
  if (!plan || !units) return MOE_EINVAL;
  return run_experts<false>(wts, opts, plan, units, units_bytes, nullptr, nullptr, B, topk, ws, ws_bytes, out,
                            out_bytes, stream);
}

int moe_decode_run(const moe_weights_t* wts, const moe_run_opts_t* opts, const void* x, const int32_t* ids,
                   int32_t B, int32_t topk, void* ws, size_t ws_bytes, void* out, size_t out_bytes, void* stream) {
  if (!x || !ids) return MOE_EINVAL;
  if (B > kDecodeMax) return run_step_grouped(wts, opts, x, ids, B, topk, ws, ws_bytes, out, out_bytes, stream);
  return run_experts<true>(wts, opts, nullptr, nullptr, 0, x, ids, B, topk, ws, ws_bytes, out, out_bytes, stream);
}

int moe_decode_run_noalloc(const moe_weights_t* wts, const moe_run_opts_t* opts, const void* x, const int32_t* ids,
                           int32_t B, int32_t topk, void* out, size_t out_bytes, void* stream) {
  if (!wts || !x || !ids || !out || B < 1 || B > kDecodeMax || topk < 1 || topk > 64) return MOE_EINVAL;
  const int E = wts->E, D = wts->D, I = wts->I;
  if (!shape_ok(E, D, I) || !wts->w13 || !wts->s13 || !wts->w2 || !wts->s2) return MOE_EINVAL;
  moe_run_opts_t o;
  std::memset(&o, 0, sizeof(o));
  if (opts) o = *opts;
  if (o.hidden_rule < 0 || o.hidden_rule > 2 || o.grid < 0 || o.col_tiles < 0 || o.col_tiles > 1 ||
      (o.ring != 0 && (o.ring < 2 || o.ring > 4)) || o.exchange != 0 || o.fc2_claims < 0 || o.fc2_claims > 1 ||
      !pf_ok(o) || ((o.hidden_codes_dev == nullptr) != (o.hidden_scales_dev == nullptr)) ||
      (o.plan_bytes != 0 && o.plan_dev == nullptr))
    return MOE_EINVAL;
  if (out_bytes < static_cast<size_t>(B) * topk * D * 2) return MOE_ENOSPACE;
  if (o.plan_dev != nullptr && o.plan_bytes < static_cast<size_t>(B) * D / 32 * 33) return MOE_ENOSPACE;
  // the scratch holds the whole-K form's exchange for at most kQGMax distinct experts of
  // at most 8 token columns and I <= 512; the kernel's own limits are the same
  if (!whole_fits(wts, B, topk)) return MOE_ELIMIT;
  uint8_t* base = scratch_ptr();
  if (base == nullptr) return MOE_EHIP;
  return launch_decode_whole(wts, o, x, ids, B, topk, reinterpret_cast<uint32_t*>(base + kScratchCalls),
                             reinterpret_cast<uint64_t*>(base + kScratchClaims),
                             reinterpret_cast<int32_t*>(base + kScratchStatus),
                             reinterpret_cast<uint64_t*>(base + kScratchHq), out, stream);
}

}  // extern "C"
