// moe_mx.hip -- MI355X (gfx950) routed-experts MoE decode step: MXFP8 activations x
// FP4 (e2m1 + E8M0) expert weights, behind the C ABI of include/moe_mx.h.
//
// Sources (vLLM API documentation pages):
//   [experts]  "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.moe.experts"
//   [runtime]  "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.moe.experts_runtime"
// The pages' engine (TMA producer warp, TMEM accumulators, mbarriers, clusters) is
// NVIDIA-specific; this file keeps the method (MXFP8 plan, (expert, <=8 token) units,
// FC1 -> gated activation -> hidden requant -> FC2, rows in top-k order, claim-based
// work distribution) and maps it onto CDNA4:
//   * weights stream from HBM once per distinct expert per call with 128-bit loads
//     straight into the operand registers of v_mfma_scale_f32_16x16x128_f8f6f4
//     (FP4 A operand = a 16-row weight tile, FP8 B operand = 16 token columns);
//   * block scales go to the MFMA as E8M0 operands (no dequantization pass);
//   * one persistent kernel claims work items in order from a device-wide counter:
//     FC1 items first, then FC2 items that wait on their expert's hidden, which only
//     earlier-claimed FC1 items produce -- no co-residency is needed;
//   * the FC1->FC2 hidden exchange and the FC1 split-K partial sums cross XCDs
//     through device-coherent (sc1) stores/loads plus agent-scope atomics.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "moe_mx.h"

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWG = 256;          // threads per experts workgroup (4 waves)
constexpr int kHBMax = 128;       // hidden blocks of 32 per expert (I <= 4096)
constexpr int kFC2Rows = 256;     // output rows per FC2 work item (4 tiles per wave)
constexpr int kGroupThreads = 1024;
constexpr uint32_t kSpinLimit = 1u << 22;  // polls of a flag before giving up

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
__device__ __forceinline__ v8i fp8_operand(uint4 lo, uint4 hi) {
  v8i r = {static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z), static_cast<int>(lo.w),
           static_cast<int>(hi.x), static_cast<int>(hi.y), static_cast<int>(hi.z), static_cast<int>(hi.w)};
  return r;
}

// ------------------------------------------------------------------ plan
// One thread per 32-element block of a token row (experts page, plan_chunk: the same
// quantization as mx_block).  x: BF16 [B, D]; codes [B, D]; scales [B, D/32].
__global__ __launch_bounds__(256) void plan_kernel(const uint8_t* __restrict__ x, int64_t nblocks,
                                                   uint8_t* __restrict__ codes,
                                                   uint8_t* __restrict__ scales) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= nblocks) return;
  const uint8_t* src = x + idx * 64;
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 q = ld16(src + 16 * i);
    w[4 * i + 0] = q.x; w[4 * i + 1] = q.y; w[4 * i + 2] = q.z; w[4 * i + 3] = q.w;
  }
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
  uint32_t c[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
    c[k] = to_e4m3(v[4 * k] * s) | (to_e4m3(v[4 * k + 1] * s) << 8) |
           (to_e4m3(v[4 * k + 2] * s) << 16) | (to_e4m3(v[4 * k + 3] * s) << 24);
  uint4* dst = reinterpret_cast<uint4*>(codes + idx * 32);
  dst[0] = make_uint4(c[0], c[1], c[2], c[3]);
  dst[1] = make_uint4(c[4], c[5], c[6], c[7]);
  scales[idx] = static_cast<uint8_t>(e + 127);
}

// ------------------------------------------------------------------ workspace
struct Table {
  int32_t* hdr;          // [16]: n_units, n_groups, n_tiles, flags (1: id out of range,
                         //        2: id repeated in a token, 4: a hidden wait timed out)
  int32_t* unit_expert;  // [U]
  int32_t* unit_rows;    // [U, 8]
  int32_t* g_expert;     // [G]
  int32_t* g_unit0;      // [G]
  int32_t* g_nunits;     // [G]
  int32_t* g_tile0;      // [G]
};

struct Layout {
  size_t ready, arrive, hdr, unit_expert, unit_rows, g_expert, g_unit0, g_nunits, g_tile0;
  size_t hcodes, hscales, partials, end;
  int64_t max_tiles;
};

constexpr size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

// Offsets depend only on (E, B, topk) up to the table, so moe_group and
// moe_experts_run agree; the counters live in a region sized by E alone, which every
// experts call leaves zero.
Layout make_layout(int E, int B, int K, int I, int S) {
  Layout L{};
  const int64_t U = static_cast<int64_t>(B) * K;
  const int64_t G = U < E ? U : E;
  size_t off = 256;  // control words: [0] claim counter, [1] done counter
  L.ready = off;
  off += static_cast<size_t>(E) * 4;
  L.arrive = off;
  off = align256(off + static_cast<size_t>(E) * kHBMax * 4);
  L.hdr = off;
  off += 64;
  L.unit_expert = off;
  off += U * 4;
  L.unit_rows = off;
  off += U * 32;
  L.g_expert = off;
  off += G * 4;
  L.g_unit0 = off;
  off += G * 4;
  L.g_nunits = off;
  off += G * 4;
  L.g_tile0 = off;
  off = align256(off + G * 4);
  L.max_tiles = (U + 15 * G + 15) / 16;
  if (I > 0) {
    const int64_t IP = (I + 127) / 128 * 128;
    L.hcodes = off;
    off = align256(off + L.max_tiles * 16 * IP);
    L.hscales = off;
    off = align256(off + L.max_tiles * 16 * (IP / 32));
    L.partials = off;
    if (S > 1) off = align256(off + L.max_tiles * (I / 32) * S * 4096);
  }
  L.end = off;
  return L;
}

Table table_at(uint8_t* ws, const Layout& L) {
  Table t;
  t.hdr = reinterpret_cast<int32_t*>(ws + L.hdr);
  t.unit_expert = reinterpret_cast<int32_t*>(ws + L.unit_expert);
  t.unit_rows = reinterpret_cast<int32_t*>(ws + L.unit_rows);
  t.g_expert = reinterpret_cast<int32_t*>(ws + L.g_expert);
  t.g_unit0 = reinterpret_cast<int32_t*>(ws + L.g_unit0);
  t.g_nunits = reinterpret_cast<int32_t*>(ws + L.g_nunits);
  t.g_tile0 = reinterpret_cast<int32_t*>(ws + L.g_tile0);
  return t;
}

// ------------------------------------------------------------------ group
// Inclusive scan of three counters over the 1024 threads of the group kernel.
struct I3 { int a, b, c; };
__device__ I3 block_scan3(I3 v, I3* wave_tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int a = __shfl_up(v.a, d), b = __shfl_up(v.b, d), c = __shfl_up(v.c, d);
    if (lane >= d) { v.a += a; v.b += b; v.c += c; }
  }
  if (lane == 63) wave_tot[wave] = v;
  __syncthreads();
  I3 base = {0, 0, 0};
  for (int w = 0; w < wave; ++w) { base.a += wave_tot[w].a; base.b += wave_tot[w].b; base.c += wave_tot[w].c; }
  v.a += base.a; v.b += base.b; v.c += base.c;
  return v;
}

// One workgroup builds the unit table (experts page, ExpertsKernel.group /
// ExpertsGroupKernel): per-expert token bitmasks, ceil(n/8) units per expert numbered
// in expert order, unit rows holding pair indices in token order (-1 padded), and the
// list of distinct experts with their first unit and 16-column tile offset.
__global__ __launch_bounds__(kGroupThreads) void group_kernel(const int32_t* __restrict__ ids, int B,
                                                              int K, int E, int W, Table tbl) {
  extern __shared__ uint32_t lds[];
  uint32_t* masks = lds;                                        // [E, W]
  int* routes = reinterpret_cast<int*>(masks + static_cast<size_t>(E) * W);  // [E] route counts
  int* unit0 = routes + E;                                      // [E]
  __shared__ I3 wave_tot[kGroupThreads / 64];
  __shared__ int flags;
  const int tid = threadIdx.x;
  const int U = B * K;
  for (int i = tid; i < E * W; i += kGroupThreads) masks[i] = 0;
  for (int i = tid; i < E; i += kGroupThreads) routes[i] = 0;
  if (tid == 0) flags = 0;
  __syncthreads();
  for (int r = tid; r < U; r += kGroupThreads) {
    const int e = ids[r];
    if (e < 0 || e >= E) { atomicOr(&flags, 1); continue; }
    const int t = r / K;
    atomicOr(&masks[e * W + (t >> 5)], 1u << (t & 31));
    atomicAdd(&routes[e], 1);
  }
  __syncthreads();
  int cnt = 0;
  if (tid < E)
    for (int w = 0; w < W; ++w) cnt += __popc(masks[tid * W + w]);
  if (tid < E && cnt != routes[tid]) atomicOr(&flags, 2);      // an id repeated in a token
  const int units = (cnt + 7) >> 3;
  I3 v = {units, cnt > 0 ? 1 : 0, (units + 1) >> 1};
  const I3 inc = block_scan3(v, wave_tot);
  const int u0 = inc.a - v.a, gi = inc.b - v.b, t0 = inc.c - v.c;
  if (tid < E) unit0[tid] = u0;
  if (tid < E && cnt > 0) {
    tbl.g_expert[gi] = tid;
    tbl.g_unit0[gi] = u0;
    tbl.g_nunits[gi] = units;
    tbl.g_tile0[gi] = t0;
    for (int u = 0; u < units; ++u) tbl.unit_expert[u0 + u] = tid;
    for (int s = cnt & 7; s != 0 && s < 8; ++s) tbl.unit_rows[(u0 + units - 1) * 8 + s] = -1;
  }
  __syncthreads();
  if (tid == kGroupThreads - 1) {
    tbl.hdr[0] = inc.a;
    tbl.hdr[1] = inc.b;
    tbl.hdr[2] = inc.c;
    tbl.hdr[3] = flags;
  }
  for (int r = tid; r < U; r += kGroupThreads) {
    const int e = ids[r];
    if (e < 0 || e >= E) continue;
    const int t = r / K;
    const uint32_t* m = masks + e * W;
    int rank = __popc(m[t >> 5] & ((1u << (t & 31)) - 1u));
    for (int w = 0; w < (t >> 5); ++w) rank += __popc(m[w]);
    tbl.unit_rows[(unit0[e] + (rank >> 3)) * 8 + (rank & 7)] = r;
  }
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

// Packed FC1 scales: per (e, j, group q of four K steps, tile rt, lane l) one word whose
// byte i is the E8M0 of (row, K-block 4*(4q+i) + l/16).
__global__ void pack_w13_scales(const uint8_t* __restrict__ src, uint32_t* __restrict__ dst, int E, int D,
                                int I) {
  const int HB = I / 32, NS = D / 128, NQ = (NS + 3) / 4;
  const int64_t total = static_cast<int64_t>(E) * HB * NQ * 256;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= total) return;
  const int l = idx & 63, rt = (idx >> 6) & 3;
  const int64_t rest = idx >> 8;
  const int q = rest % NQ;
  const int j = (rest / NQ) % HB;
  const int e = rest / (static_cast<int64_t>(NQ) * HB);
  const int r = w13_row(I, j, rt, l);
  uint32_t word = 0;
  for (int i = 0; i < 4; ++i) {
    const int s = 4 * q + i;
    const uint32_t b = s < NS ? src[(static_cast<int64_t>(e) * 2 * I + r) * (D / 32) + 4 * s + (l >> 4)] : 127u;
    word |= b << (8 * i);
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
struct ExpArgs {
  const uint8_t* w13p;
  const uint8_t* s13p;
  const uint8_t* w2p;
  const uint8_t* s2p;
  const uint8_t* xcodes;
  const uint8_t* xscales;
  uint32_t* ctrl;
  uint32_t* ready;
  uint32_t* arrive;
  Table tbl;
  uint8_t* hcodes;
  uint8_t* hscales;
  float* partials;
  uint16_t* out;
  uint8_t* dump_codes;
  uint8_t* dump_scales;
  int D, I, HB, NS1, NQ1, NS2, IP, K, S, floor_rule;
};

// Pair index (t*topk + s) of column `col` of an expert group, or -1 (padding).
__device__ __forceinline__ int column_pair(const ExpArgs& a, int unit0, int nunits, int col) {
  const int u = col >> 3;
  return u < nunits ? a.tbl.unit_rows[(unit0 + u) * 8 + (col & 7)] : -1;
}

// Gated activation and MXFP8 requantization of one 16-column tile of hidden block j
// (experts page, ExpertsKernel.store_hidden: SwiGLU here, FP32 hidden straight from
// the accumulators, one E8M0 exponent per 32 hidden values of a route).
// tot[0], tot[1]: gate rows 0-15 / 16-31 of the block; tot[2], tot[3]: the matching
// up rows.  Lane l holds column l%16, block rows 4*(l/16)+r (+16 for tot[1], tot[3]).
// Called by one whole wave.
__device__ void hidden_epilogue(const ExpArgs& a, const v4f (&tot)[4], int j, int gtile, int pair) {
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
  uint8_t* hc = a.hcodes + static_cast<int64_t>(gcol) * a.IP + 32 * j + 4 * (l >> 4);
  st_dev_u32(hc, word[0]);
  st_dev_u32(hc + 16, word[1]);
  if (l < 16) st_dev_u8(a.hscales + static_cast<int64_t>(gcol) * (a.IP / 32) + j, static_cast<uint8_t>(e + 127));
  if (a.dump_codes != nullptr && pair >= 0) {
    uint8_t* dc = a.dump_codes + static_cast<int64_t>(pair) * a.I + 32 * j + 4 * (l >> 4);
    *reinterpret_cast<uint32_t*>(dc) = word[0];
    *reinterpret_cast<uint32_t*>(dc + 16) = word[1];
    if (l < 16) a.dump_scales[static_cast<int64_t>(pair) * (a.I / 32) + j] = static_cast<uint8_t>(e + 127);
  }
}

// FC1 work item: hidden block j (gate and up rows: four 16-row tiles) of the item's
// expert over the K-step groups [q_lo, q_hi) (split c of S), for every token of the
// expert (16-column tiles, NT at a time).  Wave w takes the K steps s = 4q + w, so each
// wave streams its own contiguous KB runs; the four waves' partial sums are reduced
// through LDS in a fixed order.  With S > 1 the split sums meet in the workspace and
// the last-arriving split finishes the block (deterministic: splits summed in order).
template <int NT, int QMAX>
__device__ void fc1_item(const ExpArgs& a, int item, float* red) {
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int per_g = a.HB * a.S;
  const int g = item / per_g, rem = item - g * per_g;
  const int j = rem / a.S, c = rem - j * a.S;
  const int e = a.tbl.g_expert[g], unit0 = a.tbl.g_unit0[g], nunits = a.tbl.g_nunits[g];
  const int tile0 = a.tbl.g_tile0[g];
  const int ntiles = (nunits + 1) >> 1;
  const int q_lo = c * a.NQ1 / a.S, q_hi = (c + 1) * a.NQ1 / a.S, nq = q_hi - q_lo;
  const uint8_t* wbase = a.w13p + static_cast<int64_t>(e * a.HB + j) * a.NS1 * 4096 + l * 16;
  const uint8_t* sbase = a.s13p + static_cast<int64_t>(e * a.HB + j) * a.NQ1 * 1024 + l * 4;
  const int xrow_scales = a.D / 32;

  for (int cb = 0; cb < ntiles; cb += NT) {
    int tok[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int pair = (cb + n < ntiles) ? column_pair(a, unit0, nunits, (cb + n) * 16 + (l & 15)) : -1;
      tok[n] = pair >= 0 ? pair / a.K : -1;
    }
    v4f acc[4][NT];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[rt][n] = v4f{0.f, 0.f, 0.f, 0.f};
    // K-step groups in chunks of QMAX: every load of a chunk is issued before its first
    // MFMA (weights from HBM, activations from L2).
    for (int qc = 0; qc < nq; qc += QMAX) {
      const int nqc = nq - qc < QMAX ? nq - qc : QMAX;
      uint4 A[QMAX][4];
      uint32_t SA[QMAX][4];
      uint4 BL[QMAX][NT], BH[QMAX][NT];
      uint32_t SB[QMAX][NT];
#pragma unroll
      for (int qi = 0; qi < QMAX; ++qi) {
        const int q = q_lo + qc + (qi < nqc ? qi : nqc - 1);
        const int s = 4 * q + w;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          A[qi][rt] = ld16(wbase + (static_cast<int64_t>(s) * 4 + rt) * 1024);
          SA[qi][rt] = ld4(sbase + (static_cast<int64_t>(q) * 4 + rt) * 256);
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const int t = tok[n] >= 0 ? tok[n] : 0;
          const uint8_t* xr = a.xcodes + static_cast<int64_t>(t) * a.D + s * 128 + 16 * (l >> 4);
          BL[qi][n] = ld16(xr);
          BH[qi][n] = ld16(xr + 64);
          SB[qi][n] = ld4(a.xscales + static_cast<int64_t>(t) * xrow_scales + 4 * s);
        }
      }
#pragma unroll
      for (int qi = 0; qi < QMAX; ++qi) {
        if (qi < nqc) {
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            const bool live = tok[n] >= 0;
            const uint4 z = make_uint4(0, 0, 0, 0);
            const v8i b = fp8_operand(live ? BL[qi][n] : z, live ? BH[qi][n] : z);
            const int sb = live ? static_cast<int>((SB[qi][n] >> (8 * (l >> 4))) & 0xffu) : 127;
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
              const int sa = static_cast<int>((SA[qi][rt] >> (8 * w)) & 0xffu);
              acc[rt][n] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                  fp4_operand(A[qi][rt]), b, acc[rt][n], 4, 0, 0, sa, 0, sb);
            }
          }
        }
      }
    }
    // Cross-wave reduction: waves 1..3 park their sums in LDS, wave 0 adds them in order.
    if (w > 0) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int n = 0; n < NT; ++n)
          *reinterpret_cast<v4f*>(red + ((((w - 1) * 4 + rt) * NT + n) * 64 + l) * 4) = acc[rt][n];
    }
    __syncthreads();
    if (w == 0) {
#pragma unroll
      for (int ww = 0; ww < 3; ++ww)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
          for (int n = 0; n < NT; ++n)
            acc[rt][n] += *reinterpret_cast<const v4f*>(red + (((ww * 4 + rt) * NT + n) * 64 + l) * 4);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        if (cb + n >= ntiles) continue;
        const int gtile = tile0 + cb + n;
        if (a.S == 1) {
          const v4f tot[4] = {acc[0][n], acc[1][n], acc[2][n], acc[3][n]};
          const int pair = column_pair(a, unit0, nunits, (cb + n) * 16 + (l & 15));
          hidden_epilogue(a, tot, j, gtile, pair);
        } else {
          float* p = a.partials + ((static_cast<int64_t>(gtile) * a.HB + j) * a.S + c) * 1024 + l * 4;
#pragma unroll
          for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r) st_dev_u32(p + rt * 256 + r, __float_as_uint(acc[rt][n][r]));
        }
      }
    }
    __syncthreads();
  }

  if (w != 0) return;
  if (a.S > 1) {
    wait_stores();
    uint32_t old = 0;
    if (l == 0)
      old = __hip_atomic_fetch_add(a.arrive + g * kHBMax + j, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old != static_cast<uint32_t>(a.S - 1)) return;   // another split finishes the block
    compiler_fence();
    if (l == 0) st_dev_u32(a.arrive + g * kHBMax + j, 0u);  // re-arm for the next call
    for (int t = 0; t < ntiles; ++t) {
      const int gtile = tile0 + t;
      v4f tot[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) tot[rt] = v4f{0.f, 0.f, 0.f, 0.f};
      for (int cc = 0; cc < a.S; ++cc) {
        const float* p = a.partials + ((static_cast<int64_t>(gtile) * a.HB + j) * a.S + cc) * 1024 + l * 4;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const uint64_t lo = ld_dev_u64(p + rt * 256), hi = ld_dev_u64(p + rt * 256 + 2);
          tot[rt][0] += __uint_as_float(static_cast<uint32_t>(lo));
          tot[rt][1] += __uint_as_float(static_cast<uint32_t>(lo >> 32));
          tot[rt][2] += __uint_as_float(static_cast<uint32_t>(hi));
          tot[rt][3] += __uint_as_float(static_cast<uint32_t>(hi >> 32));
        }
      }
      const int pair = column_pair(a, unit0, nunits, t * 16 + (l & 15));
      hidden_epilogue(a, tot, j, gtile, pair);
    }
  }
  // Publish: the hidden block's codes and scale are stored (sc1) before the count.
  wait_stores();
  if (l == 0) __hip_atomic_fetch_add(a.ready + g, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// FC2 work item: 256 output rows (16 tiles; wave w takes tiles w, w+4, w+8, w+12) of
// one expert for all its tokens.  The weight loads are issued before waiting for the
// expert's hidden, so the wait overlaps the stream.  Output: BF16 rows
// out[pair, d] (experts page, ExpertsKernel.fc2: rows of the unit's pair indices).
template <int NT>
__device__ void fc2_item(const ExpArgs& a, int item) {
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int RB = a.D / kFC2Rows;
  const int g = item / RB, rb = item - g * RB;
  const int e = a.tbl.g_expert[g], unit0 = a.tbl.g_unit0[g], nunits = a.tbl.g_nunits[g];
  const int tile0 = a.tbl.g_tile0[g];
  const int ntiles = (nunits + 1) >> 1;
  const int tiles_per_expert = a.D / 16;
  uint4 A[4][4];
  uint32_t SA[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rt2 = rb * 16 + w + 4 * i;
    const int64_t tile = static_cast<int64_t>(e) * tiles_per_expert + rt2;
    const uint8_t* base = a.w2p + tile * a.NS2 * 1024 + l * 16;
#pragma unroll
    for (int s = 0; s < 4; ++s) A[i][s] = ld16(base + (s < a.NS2 ? s : a.NS2 - 1) * 1024);
    SA[i] = ld4(a.s2p + tile * 256 + l * 4);
  }
  // Wait until every hidden block of this expert is published (FC1 items of the
  // expert were claimed before this item, so they are running or done).
  // The wait is bounded (seconds) so that a broken invariant can never hang the GPU:
  // it then flags the table header (bit 2) and computes with whatever is there.
  for (uint32_t spins = 0; ld_dev_u32(a.ready + g) < static_cast<uint32_t>(a.HB); ++spins) {
    if (spins == kSpinLimit) {
      __hip_atomic_fetch_or(a.tbl.hdr + 3, 4, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  compiler_fence();

  for (int cb = 0; cb < ntiles; cb += NT) {
    uint4 BL[NT][4], BH[NT][4];
    uint32_t SB[NT][4];
    bool live[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      live[n] = cb + n < ntiles;
      const int gcol = (tile0 + (live[n] ? cb + n : 0)) * 16 + (l & 15);
      const uint8_t* hc = a.hcodes + static_cast<int64_t>(gcol) * a.IP + 16 * (l >> 4);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int ss = s < a.NS2 ? s : a.NS2 - 1;
        const uint64_t l0 = ld_dev_u64(hc + ss * 128), l1 = ld_dev_u64(hc + ss * 128 + 8);
        const uint64_t h0 = ld_dev_u64(hc + ss * 128 + 64), h1 = ld_dev_u64(hc + ss * 128 + 72);
        BL[n][s] = make_uint4(static_cast<uint32_t>(l0), static_cast<uint32_t>(l0 >> 32),
                              static_cast<uint32_t>(l1), static_cast<uint32_t>(l1 >> 32));
        BH[n][s] = make_uint4(static_cast<uint32_t>(h0), static_cast<uint32_t>(h0 >> 32),
                              static_cast<uint32_t>(h1), static_cast<uint32_t>(h1 >> 32));
        SB[n][s] = ld_dev_u32(a.hscales + static_cast<int64_t>(gcol) * (a.IP / 32) + 4 * ss);
      }
    }
    v4f acc[4][NT];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[i][n] = v4f{0.f, 0.f, 0.f, 0.f};
    const int grp = l >> 4;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < a.NS2) {
        // K-blocks beyond I (I not a multiple of 128) are zero.
        const bool lo_ok = 4 * s + (grp >> 1) < a.HB, hi_ok = 4 * s + 2 + (grp >> 1) < a.HB;
        const bool sc_ok = 4 * s + grp < a.HB;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const uint4 z = make_uint4(0, 0, 0, 0);
          const v8i b = fp8_operand(live[n] && lo_ok ? BL[n][s] : z, live[n] && hi_ok ? BH[n][s] : z);
          const int sb = live[n] && sc_ok ? static_cast<int>((SB[n][s] >> (8 * grp)) & 0xffu) : 127;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int sa = static_cast<int>((SA[i] >> (8 * s)) & 0xffu);
            acc[i][n] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fp4_operand(A[i][s]), b, acc[i][n],
                                                                          4, 0, 0, sa, 0, sb);
          }
        }
      }
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      if (!live[n]) continue;
      const int pair = column_pair(a, unit0, nunits, (cb + n) * 16 + (l & 15));
      if (pair < 0) continue;
      uint16_t* orow = a.out + static_cast<int64_t>(pair) * a.D;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = (rb * 16 + w + 4 * i) * 16 + 4 * grp;
        const uint2 v = make_uint2(to_bf16_bits(acc[i][n][0]) | (to_bf16_bits(acc[i][n][1]) << 16),
                                   to_bf16_bits(acc[i][n][2]) | (to_bf16_bits(acc[i][n][3]) << 16));
        *reinterpret_cast<uint2*>(orow + d) = v;
      }
    }
  }
}

// The persistent routed-experts kernel (experts page, ExpertsKernel; runtime page,
// PersistentExperts.run).  Items [0, G*HB*S) are FC1 splits, [G*HB*S, +G*D/256) FC2
// row blocks, claimed in order.  The last workgroup to leave re-arms the counters.
template <int NT, int QMAX>
__global__ __launch_bounds__(kWG) void experts_kernel(ExpArgs a) {
  __shared__ float red[3 * 4 * NT * 64 * 4];
  __shared__ int s_item, s_last;
  const int n_groups = a.tbl.hdr[1];
  const int n_fc1 = n_groups * a.HB * a.S;
  const int total = n_fc1 + n_groups * (a.D / kFC2Rows);
  for (;;) {
    if (threadIdx.x == 0)
      s_item = static_cast<int>(__hip_atomic_fetch_add(a.ctrl, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    __syncthreads();
    const int item = s_item;
    __syncthreads();
    if (item >= total) break;
    if (item < n_fc1)
      fc1_item<NT, QMAX>(a, item, red);
    else
      fc2_item<NT>(a, item - n_fc1);
  }
  if (threadIdx.x == 0) {
    wait_stores();
    const uint32_t done = __hip_atomic_fetch_add(a.ctrl + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = done == gridDim.x - 1;
  }
  __syncthreads();
  if (s_last) {
    for (int i = threadIdx.x; i < n_groups; i += kWG) st_dev_u32(a.ready + i, 0u);
    if (threadIdx.x == 0) {
      st_dev_u32(a.ctrl, 0u);
      st_dev_u32(a.ctrl + 1, 0u);
    }
  }
}

using ExpertsFn = void (*)(ExpArgs);

// Kernel variants: NT column tiles per weight pass x QMAX K-step groups held in
// registers per wave (QMAX is capped so the preloaded operands stay in registers).
ExpertsFn pick_kernel(int nt, int qmax) {
  if (nt == 1) {
    if (qmax == 1) return experts_kernel<1, 1>;
    if (qmax == 2) return experts_kernel<1, 2>;
    if (qmax == 4) return experts_kernel<1, 4>;
    return experts_kernel<1, 8>;
  }
  if (nt == 2) {
    if (qmax == 1) return experts_kernel<2, 1>;
    if (qmax == 2) return experts_kernel<2, 2>;
    return experts_kernel<2, 4>;
  }
  if (qmax == 1) return experts_kernel<4, 1>;
  return experts_kernel<4, 2>;
}

// ------------------------------------------------------------------ host helpers
bool shape_ok(int64_t E, int64_t D, int64_t I) {
  return E >= 1 && E <= 1024 && D >= 512 && D <= 16384 && D % 512 == 0 && I >= 32 && I <= 512 && I % 32 == 0;
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

// Column tiles per weight pass: an expert never has more tokens than the batch.
int auto_col_tiles(int B) { return B <= 16 ? 1 : (B <= 32 ? 2 : 4); }
int qmax_cap(int nt) { return nt == 1 ? 8 : (nt == 2 ? 4 : 2); }
int max_ksplit(int B, int K, int NQ1) {
  const int cap = static_cast<int64_t>(B) * K <= 256 ? 8 : 2;
  return NQ1 < cap ? NQ1 : cap;
}
int pow2_at_least(int v) { int p = 1; while (p < v) p <<= 1; return p; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int launch_status() { return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP; }

}  // namespace

// ====================================================================== C ABI
extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument or unsupported shape";
    case MOE_ENOSPACE: return "buffer too small";
    case MOE_EHIP: return "HIP launch or runtime error";
    default: return "unknown status";
  }
}

size_t moe_plan_bytes(int32_t B, int32_t D) {
  if (B < 1 || D < 32 || D % 32) return 0;
  return static_cast<size_t>(B) * D + static_cast<size_t>(B) * (D / 32);
}

size_t moe_workspace_bytes(int32_t E, int32_t D, int32_t I, int32_t B_max, int32_t topk) {
  if (!shape_ok(E, D, I) || B_max < 1 || topk < 1 || topk > 64 || static_cast<int64_t>(B_max) * topk > 65536)
    return 0;
  const int NQ1 = D / 512;
  size_t best = 0;
  for (int b = 1; b <= B_max; ++b) {
    const size_t end = make_layout(E, b, topk, I, max_ksplit(b, topk, NQ1)).end;
    if (end > best) best = end;
  }
  return best;
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
  const int HB = I / 32, NS1 = D / 128, NQ1 = (NS1 + 3) / 4, NS2 = (I + 127) / 128, NQ2 = (NS2 + 3) / 4;
  auto blocks = [](int64_t n) { return static_cast<unsigned>((n + 255) / 256); };
  const int64_t n1 = static_cast<int64_t>(E) * HB * NS1 * 256, n2 = static_cast<int64_t>(E) * HB * NQ1 * 256;
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
  hipLaunchKernelGGL(plan_kernel, dim3(static_cast<unsigned>((nblocks + 255) / 256)), dim3(256), 0,
                     as_stream(stream), static_cast<const uint8_t*>(x), nblocks, codes,
                     codes + static_cast<int64_t>(B) * D);
  return launch_status();
}

int moe_group(const int32_t* ids, int32_t B, int32_t topk, int32_t E, void* ws, size_t ws_bytes, void* stream) {
  if (!ids || !ws || B < 1 || topk < 1 || topk > 64 || E < 1 || E > 1024 ||
      static_cast<int64_t>(B) * topk > 65536)
    return MOE_EINVAL;
  const int W = (B + 31) / 32;
  const size_t lds = (static_cast<size_t>(E) * W + 2 * static_cast<size_t>(E)) * 4;
  if (lds > 60 * 1024) return MOE_EINVAL;
  const Layout L = make_layout(E, B, topk, 0, 1);
  if (ws_bytes < L.end) return MOE_ENOSPACE;
  const Table t = table_at(static_cast<uint8_t*>(ws), L);
  hipLaunchKernelGGL(group_kernel, dim3(1), dim3(kGroupThreads), lds, as_stream(stream), ids, B, topk, E, W, t);
  return launch_status();
}

int moe_units_export(const void* ws, size_t ws_bytes, int32_t B, int32_t topk, int32_t E, void* header,
                     void* unit_expert, void* unit_rows, int32_t max_units, void* stream) {
  if (!ws || !header || !unit_expert || !unit_rows || B < 1 || topk < 1 || E < 1 || max_units < 0)
    return MOE_EINVAL;
  const Layout L = make_layout(E, B, topk, 0, 1);
  if (ws_bytes < L.end) return MOE_ENOSPACE;
  const int64_t U = static_cast<int64_t>(B) * topk;
  const int64_t n = max_units < U ? max_units : U;
  const uint8_t* base = static_cast<const uint8_t*>(ws);
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

int moe_experts_run(const moe_weights_t* wts, const moe_run_opts_t* opts, const void* plan, int32_t B,
                    int32_t topk, void* ws, size_t ws_bytes, void* out, size_t out_bytes, void* stream) {
  if (!wts || !plan || !ws || !out || B < 1 || topk < 1 || topk > 64 || static_cast<int64_t>(B) * topk > 65536)
    return MOE_EINVAL;
  const int E = wts->E, D = wts->D, I = wts->I;
  if (!shape_ok(E, D, I) || !wts->w13 || !wts->s13 || !wts->w2 || !wts->s2) return MOE_EINVAL;
  moe_run_opts_t o;
  std::memset(&o, 0, sizeof(o));
  if (opts) o = *opts;
  if (o.hidden_rule < 0 || o.hidden_rule > 2 || o.ksplit < 0 || o.grid < 0 || o.col_tiles < 0 ||
      (o.fc2_rows != 0 && o.fc2_rows != kFC2Rows) ||
      (o.col_tiles != 0 && o.col_tiles != 1 && o.col_tiles != 2 && o.col_tiles != 4) ||
      ((o.hidden_codes_dev == nullptr) != (o.hidden_scales_dev == nullptr)))
    return MOE_EINVAL;
  if (out_bytes < static_cast<size_t>(B) * topk * D * 2) return MOE_ENOSPACE;
  if (ws_bytes < make_layout(E, B, topk, I, 1).end) return MOE_ENOSPACE;  // before touching the device

  const int HB = I / 32, NS1 = D / 128, NQ1 = (NS1 + 3) / 4, NS2 = (I + 127) / 128;
  const int cus = device_cus();
  const int nt = o.col_tiles ? o.col_tiles : auto_col_tiles(B);
  const int kmax = max_ksplit(B, topk, NQ1);
  int S = o.ksplit;
  if (S == 0) {
    const int64_t groups = static_cast<int64_t>(B) * topk < E ? static_cast<int64_t>(B) * topk : E;
    const int64_t want = (3 * static_cast<int64_t>(cus) + groups * HB - 1) / (groups * HB);
    S = static_cast<int>(want < 1 ? 1 : (want > kmax ? kmax : want));
  }
  if (S > kmax) return MOE_ENOSPACE;  // the workspace holds partial sums for up to kmax splits
  int qmax = pow2_at_least((NQ1 + S - 1) / S);  // K-step groups per item, held in chunks of
  if (qmax > qmax_cap(nt)) qmax = qmax_cap(nt);   // at most qmax_cap (register budget)
  const Layout L = make_layout(E, B, topk, I, S);
  if (ws_bytes < L.end) return MOE_ENOSPACE;

  uint8_t* base = static_cast<uint8_t*>(ws);
  ExpArgs a;
  a.w13p = static_cast<const uint8_t*>(wts->w13);
  a.s13p = static_cast<const uint8_t*>(wts->s13);
  a.w2p = static_cast<const uint8_t*>(wts->w2);
  a.s2p = static_cast<const uint8_t*>(wts->s2);
  a.xcodes = static_cast<const uint8_t*>(plan);
  a.xscales = a.xcodes + static_cast<int64_t>(B) * D;
  a.ctrl = reinterpret_cast<uint32_t*>(base);
  a.ready = reinterpret_cast<uint32_t*>(base + L.ready);
  a.arrive = reinterpret_cast<uint32_t*>(base + L.arrive);
  a.tbl = table_at(base, L);
  a.hcodes = base + L.hcodes;
  a.hscales = base + L.hscales;
  a.partials = reinterpret_cast<float*>(base + L.partials);
  a.out = static_cast<uint16_t*>(out);
  a.dump_codes = static_cast<uint8_t*>(o.hidden_codes_dev);
  a.dump_scales = static_cast<uint8_t*>(o.hidden_scales_dev);
  a.D = D;
  a.I = I;
  a.HB = HB;
  a.NS1 = NS1;
  a.NQ1 = NQ1;
  a.NS2 = NS2;
  a.IP = NS2 * 128;
  a.K = topk;
  a.S = S;
  a.floor_rule = o.hidden_rule == 2 || (o.hidden_rule == 0 && I == 384);
  const int grid = o.grid ? o.grid : 2 * cus;
  hipLaunchKernelGGL(pick_kernel(nt, qmax), dim3(grid), dim3(kWG), 0, as_stream(stream), a);
  return launch_status();
}

}  // extern "C"
