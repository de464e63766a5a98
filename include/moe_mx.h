/*
 * moe_mx.h -- C ABI of the MI355X (gfx950) routed-experts MoE decode step:
 * MXFP8 activations x FP4 (e2m1 + E8M0) expert weights.
 *
 * The operation (vLLM API pages "vllm.models.kimi_k3.nvidia.specialized_decode.
 * cutedsl.moe.experts" and "...cutedsl.moe.experts_runtime", PersistentExperts.run):
 * each token's BF16 row is quantized to MXFP8 (32-element blocks, e4m3 codes and an
 * E8M0 scale); each (token, top-k slot) route then computes, against its expert's
 * weights,
 *     a   = W13[e] . x            (FC1, 2I rows: gate 0..I-1, up I..2I-1)
 *     h   = silu(gate) * up       (FP32, SwiGLU)
 *     hq  = MXFP8(h)              (32-blocks, hidden exponent rule)
 *     y   = W2[e] . hq            (FC2, D rows), rounded to BF16
 * and the result is written as output row t*topk + s (the caller's top-k order, no
 * routing weight applied).  Experts shared by several tokens stream their weights
 * once per call for all of them.
 *
 * Conventions of every entry point:
 *   - pointers named *_dev are DEVICE pointers, owned by the caller; the library
 *     allocates nothing and keeps no pointer past the call;
 *   - `stream` is a hipStream_t (NULL = the null stream); calls only enqueue work on
 *     it and never synchronize;
 *   - the return value is MOE_OK (0) or a negative moe_status; arguments are checked
 *     on the host before anything is enqueued, so an error enqueues nothing;
 *   - device-side preconditions that are NOT checked: expert ids within [0, E) and
 *     distinct within each token's top-k (out-of-range ids are skipped and flagged in
 *     the unit table, see moe_units_export).
 *
 * Canonical data layouts (row-major, bytes):
 *   x        BF16  [B, D]
 *   plan     u8    [B, D] e4m3 codes, followed by u8 [B, D/32] E8M0 scales
 *   ids      i32   [B, topk]
 *   w13      u8    [E, 2I, D/2]  two e2m1 codes per byte, low nibble = even k
 *   s13      u8    [E, 2I, D/32] E8M0 (2^(byte-127)) per 32 consecutive k of a row
 *   w2       u8    [E, D, I/2],  s2 u8 [E, D, I/32]
 *   out      BF16  [B*topk, D]
 * Supported shapes: 512 <= D <= 16384 with D % 512 == 0, 32 <= I <= 512 with
 * I % 32 == 0, 1 <= E <= 1024, 1 <= topk <= 64, 1 <= B*topk <= 65536; moe_group also
 * needs E * ceil(B/32) + 3E + C <= 15360 with C = min(E, B*topk) + ceil(B*topk/32)
 * (its per-expert token bitmasks and counts and its per-chunk column counts live in LDS).
 */
#ifndef MOE_MX_H
#define MOE_MX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moe_status {
  MOE_OK = 0,
  MOE_EINVAL = -1,       /* null pointer, bad size or unsupported shape */
  MOE_ENOSPACE = -2,     /* plan, workspace or output buffer too small */
  MOE_EHIP = -3,         /* a HIP call or kernel launch failed */
  MOE_ELIMIT = -4,       /* moe_decode_run_noalloc: the batch needs more than its fixed scratch */
};

/* Human-readable name of a moe_status value (static string). */
const char* moe_status_string(int status);

/* ---------------------------------------------------------------- sizes ---- */

/* Bytes of the MXFP8 plan of B tokens of D features: B*D codes + B*D/32 scales
 * (experts page, ExpertsPlanKernel / plan_chunk).  0 on invalid sizes. */
size_t moe_plan_bytes(int32_t B, int32_t D);

/* Bytes of the unit-table buffer of a batch of B tokens with topk routes each over E
 * experts (experts page, ExpertsKernel.group: the per-batch grouping of routes by
 * expert): header, per-unit expert and pair rows, the distinct-expert list and the
 * 32-column chunk table.  Sized for the worst case of the batch, so one buffer serves
 * any ids.  0 on invalid sizes. */
size_t moe_units_bytes(int32_t B, int32_t topk, int32_t E);

/* Bytes of the caller-owned workspace of the experts kernel for calls with up to B_max
 * tokens (runtime page, scratch()): call counters, hidden-block flags and arrival
 * counters, the hidden-exchange images, the FC1 partial sums, and the plan the one-launch
 * grouped form (moe_decode_run, B > 8) makes with its per-workgroup flags.  Its layout is a
 * function of (E, D, I, topk) and its size, so one workspace serves every batch up to
 * the B_max it was sized for.  0 on invalid sizes. */
size_t moe_workspace_bytes(int32_t E, int32_t D, int32_t I, int32_t B_max, int32_t topk);

/* The static work split of one experts launch, evaluated on the host (no device call;
 * for checking schedules on any machine).  It is the persistent grid's division of the
 * work among its workgroups (experts page, ExpertsKernel: each CTA's FC1 blocks and
 * its FC2 tile range, and with steal the claimable zone at the end of that range).
 * form 0: the decode form's whole-K kernel, `groups` distinct experts (<= 128, I <=
 * 512); form 1: the grouped form, `groups` chunks of up to 32 routes of one expert (<=
 * 1024).  An FC1 item is one 32-wide hidden block of one group; there are groups * I/32
 * of them, and item i goes to workgroup i mod grid.  FC2 tiles are the 16-row output
 * tiles, groups * D/16 of them in group-major order, in equal runs (the grouped form's
 * three-call launch balances its runs on bytes instead: moe_grouped_runs).  claims_ring: 0, or (form 0) the
 * slots per wave (2..4) of a launch with FC2 tail claims, whose zones it then reports.
 * Outputs are host pointers:
 *   split i32 [grid, 6]: per workgroup {FC1 items, first FC2 tile, FC2 tiles, streaming
 *     waves per workgroup, first tile of its claimable zone, grains of eight tiles in it};
 *   items i32 [groups * I/32, 2] (may be NULL): (group, hidden block) of item i.
 * MOE_EINVAL for a bad form, shape, group count, grid (1..2048) or claims_ring. */
int moe_work_split(int32_t form, int32_t groups, int32_t D, int32_t I, int32_t grid, int32_t claims_ring,
                   int32_t* split, int32_t* items);

/* The FC2 runs of the grouped form as moe_experts_run's three-call form sets them (no
 * device call).  The experts page gives each CTA a contiguous share of the FC2 stream
 * (ExpertsKernel.partition); here the shares are balanced on the bytes a 16-row tile
 * moves rather than on tile counts: its FP4 weights and scales, 16 (I/2 + I/32) bytes,
 * and its BF16 output rows, 32 bytes per live column of its chunk.  Run c starts at the
 * first tile whose cost-so-far reaches floor(W c / grid), W the total.  The one-launch
 * form (moe_decode_run, B > 8) keeps equal tile counts (moe_work_split, form 1).
 * chunk_cols: host i32 [chunks], the live columns of each chunk (1..32, chunks of one
 * expert consecutive, as moe_group orders them); runs: host i32 [grid, 2], per
 * workgroup {first FC2 tile, FC2 tiles}.  MOE_EINVAL for chunks outside 0..1024, a count
 * outside 1..32 or more than 65536 columns in all, an unsupported shape or I > 384, a
 * grid outside 1..2048, or a NULL pointer. */
int moe_grouped_runs(int32_t chunks, const int32_t* chunk_cols, int32_t D, int32_t I, int32_t grid,
                     int32_t* runs);

/* Bytes of the four packed weight buffers written by moe_pack_weights (experts page,
 * ExpertsKernel.schedule / produce: the weights stream tile by tile, 128 K at a time).
 * They equal the canonical sizes (the packing only reorders 16-byte code runs and scale
 * bytes), except that FC2 codes and scales are padded to a multiple of 128 along I.
 * The four size_t outputs are host pointers (any may be NULL).  Returns MOE_OK or
 * MOE_EINVAL for an unsupported shape. */
int moe_packed_weight_bytes(int32_t E, int32_t D, int32_t I, size_t* w13_bytes,
                            size_t* s13_bytes, size_t* w2_bytes, size_t* s2_bytes);

/* ---------------------------------------------------------------- setup ---- */

/* One-time, untimed re-layout of canonical expert weights (layouts above) into the
 * tile-major order the experts kernel streams: per 16-row tile and 128-wide K step, one
 * contiguous 1 KB run of FP4 codes, and per tile the E8M0 bytes of four K steps in one
 * 32-bit word per lane (the pages likewise keep their scales tile-major, experts page
 * ExpertsKernel.schedule / produce).  All eight pointers are device buffers of the
 * sizes above; canonical and packed buffers must not overlap. */
int moe_pack_weights(int32_t E, int32_t D, int32_t I, const void* w13_dev, const void* s13_dev,
                     const void* w2_dev, const void* s2_dev, void* w13p_dev, void* s13p_dev,
                     void* w2p_dev, void* s2p_dev, void* stream);

/* Zero the workspace once after allocating it (runtime page, scratch(): the pages
 * pre-fill theirs with a sentinel).  The experts kernel keeps it consistent from call
 * to call (arrival counters re-armed, flags tagged with the call number), so no
 * per-call reset is needed. */
int moe_workspace_init(void* ws_dev, size_t ws_bytes, void* stream);

/* Packed expert weights of one layer (pointers from moe_pack_weights). */
typedef struct {
  int32_t E, D, I;
  const void* w13; /* packed FC1 codes   */
  const void* s13; /* packed FC1 scales  */
  const void* w2;  /* packed FC2 codes   */
  const void* s2;  /* packed FC2 scales  */
} moe_weights_t;

/* ----------------------------------------------------------- hot path ---- */

/* MXFP8 quantization of x (BF16 [B, D]) into `plan` (experts page, plan_chunk /
 * mx_block): per 32-element block, exact amax; E8M0 exponent e = the smallest with
 * amax * 2^-e <= 448 (0 -> e = -127); codes = e4m3 round-to-nearest-even of
 * x * 2^-e.  plan_bytes must be >= moe_plan_bytes(B, D). */
int moe_plan(const void* x_dev, int32_t B, int32_t D, void* plan_dev, size_t plan_bytes,
             void* stream);

/* Unit table of the batch's routes (experts page, ExpertsKernel.group and
 * ExpertsGroupKernel): expert e's routes, in token order, fill ceil(n_e / 8) units
 * numbered in ascending expert order; each unit row holds eight pair indices
 * t*topk + s, -1 where padded.  Also lists the distinct experts ("groups") with their
 * first unit, unit count and first 16-column tile, and cuts each expert's routes, in the
 * same order, into chunks of 32 (the grouped kernel's weight-pass width): per chunk its
 * expert, its live columns and the live columns before it, and 32 pair indices (-1
 * padded), in ascending expert order.
 * Written into `units_dev` (moe_units_bytes(B, topk, E) bytes); run it before
 * moe_experts_run on the same stream. */
int moe_group(const int32_t* ids_dev, int32_t B, int32_t topk, int32_t E, void* units_dev,
              size_t units_bytes, void* stream);

/* moe_plan and moe_group of one batch in a single launch (experts page, plan_chunk and
 * ExpertsKernel.group; the same outputs, bit for bit):
 * x_dev BF16 [B, D] -> plan_dev (moe_plan layout), ids_dev i32 [B, topk] -> units_dev
 * (moe_group layout).  Eight workgroups build the unit table while the others quantize
 * x, which saves a launch per step of the grouped form.  Arguments and errors as the two
 * calls. */
int moe_plan_group(const void* x_dev, const int32_t* ids_dev, int32_t B, int32_t D, int32_t topk, int32_t E,
                   void* plan_dev, size_t plan_bytes, void* units_dev, size_t units_bytes, void* stream);

/* Copy the unit table that moe_group wrote (experts page, ExpertsKernel.group) into
 * caller device buffers (for inspection): header_dev i32[4] = {n_units, n_groups, n_column_tiles, flags (bit 0: an
 * id was out of range, bit 1: an id repeated within a token, bit 2: an experts call gave
 * up waiting for a hidden block -- never expected)}, unit_expert_dev i32[max_units],
 * unit_rows_dev i32[max_units, 8].  Enqueued device-to-device copies. */
int moe_units_export(const void* units_dev, size_t units_bytes, int32_t B, int32_t topk, int32_t E,
                     void* header_dev, void* unit_expert_dev, void* unit_rows_dev,
                     int32_t max_units, void* stream);

/* One row of a next-layer prefetch table (runtime page, PersistentExperts.run's ahead
 * table of (address, bytes) rows): device memory the next launch will read. */
typedef struct {
  const void* addr;  /* device address, 16-byte aligned */
  uint64_t bytes;    /* below 2^31 */
} moe_prefetch_row_t;

/* Options of moe_experts_run (zero-initialise for the defaults). */
typedef struct {
  /* Exponent rule of the hidden requantization: 0 = default (the pages' choice: floor
   * on the TP8 shard, I == 384; the no-saturation rule otherwise), 1 = no saturation
   * (smallest e with amax * 2^-e <= 448), 2 = floor (OCP: e = floor(log2 amax) - 8,
   * saturating). */
  int32_t hidden_rule;
  int32_t grid;       /* persistent workgroups, at most the device's resident capacity
                         for the kernel variant (MOE_EINVAL above it); 0 = all of it */
  int32_t col_tiles;  /* moe_experts_run: 16-token column tiles per weight pass.
                         0 = default: the grouped kernel (two tiles, 32-route chunks) when
                         the batch fits its limits (I <= 384, at most 1024 chunks and 32
                         FC1 blocks per workgroup), else 1;
                         1 = the one-tile experts kernel (any batch);
                         2 = the grouped kernel only (MOE_EINVAL beyond its limits);
                         moe_decode_run: 0 or 1; other values MOE_EINVAL */
  int32_t ring;       /* weight items in flight per streaming wave (2..4) of the one-tile
                         and decode kernels; 0 = the deepest that fits in LDS next to the
                         unit table (the grouped kernel always keeps three) */
  int32_t exchange;   /* moe_decode_run only: how FC1 results reach FC2 --
                         0 = whole-K blocks (default): a hidden block's FC1 runs over all of
                         K in one workgroup, which applies SwiGLU and MXFP8 and publishes the
                         block as call-tagged (code word, call) pairs; batches beyond its
                         limits (more than 128 distinct experts, more than 576 routes, I >
                         512, B*D/32 > 2304) fall back to 2;
                         1 = call-tagged FC1 partial sums that every FC2 workgroup reduces
                         itself;
                         2 = finished split blocks (the owner of a block's first step adds
                         the other owners' partial sums, applies SwiGLU and MXFP8, publishes
                         codes and a call-tagged flag);
                         other values MOE_EINVAL */
  int32_t fc2_claims;  /* the decode form's whole-K kernel (exchange 0): 0 = default,
                         static FC2 runs; 1 = FC2 tail claims -- the last grains of eight
                         FC2 tiles of each workgroup's run are handed out through a
                         call-tagged counter of that workgroup, to itself from the front
                         and to the two workgroups before it in tile order from the back
                         where they hold that expert's hidden.  The rows are the same bit
                         for bit either way.  Other values MOE_EINVAL */
  int32_t reserved[2];
  void* hidden_codes_dev;  /* optional u8 [B*topk, I]: the hidden's e4m3 codes per route */
  void* hidden_scales_dev; /* optional u8 [B*topk, I/32]: its E8M0 scales */
  /* moe_decode_run only (MOE_EINVAL for moe_experts_run when set): */
  void* plan_dev;          /* optional: the MXFP8 plan of x the call computed, in the moe_plan
                              layout (B*D codes, then B*D/32 scales) */
  size_t plan_bytes;       /* size of plan_dev (>= B*D/32*33, else MOE_ENOSPACE) */
  int32_t* status_dev;     /* optional i32 status word the call ORs flags into: bit 0 an id out
                              of range (skipped), bit 1 an id repeated within a token (one of
                              its routes is lost), bit 2 a wait gave up (never expected).
                              NULL: the flags go to a word of the workspace. */
  /* moe_decode_run's whole-K kernel only (MOE_EINVAL elsewhere): next-layer weight
   * prefetch (runtime page, run(x, ids, weights, ahead)).  A HOST array of up to 64 rows
   * of device memory the next launch will read, typically its expert weights.  The
   * kernel splits the rows' bytes over its workgroups; each workgroup's finisher wave,
   * idle once its FC1 blocks are published, reads its share once through LDS, so that
   * the bytes sit in the Infinity Cache when that launch starts.  The rows are read, never
   * written, and change nothing this call computes; their memory must stay allocated
   * until the call has run.  The table itself is copied into the launch: it may be freed
   * when the call returns.  NULL with 0 rows: no prefetch.  MOE_EINVAL for more than 64
   * rows, a NULL table with rows, a row of 2^31 bytes or more, or a row not 16-byte
   * aligned. */
  const moe_prefetch_row_t* ahead;
  int32_t ahead_rows;
} moe_run_opts_t;

/* The routed experts (experts page, ExpertsKernel; runtime page, PersistentExperts.run):
 * FC1 against the packed w13 for every distinct expert of the batch and all of its
 * tokens, SwiGLU, MXFP8 requantization of the hidden, FC2 against the packed w2, BF16
 * rows into out_dev [B*topk, D] in the caller's top-k order.  Reads the plan written by
 * moe_plan and the unit table written by moe_group (same B and topk).
 * One persistent, co-resident kernel.  By default (col_tiles 0) the grouped kernel: an
 * FC1 work item is one 32-wide hidden block of one 32-route chunk over the whole of K,
 * so one workgroup applies SwiGLU and MXFP8 to it and publishes it (device-coherent
 * stores, a call-tagged flag); FC2 tiles are dealt as contiguous runs balanced on the
 * bytes they move (moe_grouped_runs), and each chunk's FC2 waits for its hidden blocks.  The one-tile experts kernel (col_tiles 1) instead
 * gives every workgroup an equal contiguous slice of the FC1 weight stream, then of the
 * FC2 weight stream, and FC2 waits per expert for the split blocks FC1 slices publish.
 * The grid is sized from the kernel's occupancy so that it is resident at once; do not
 * run other kernels on the device concurrently with it.  Calls that share a workspace
 * must not overlap (one stream, or ordered streams). */
int moe_experts_run(const moe_weights_t* weights, const moe_run_opts_t* opts,
                    const void* plan_dev, const void* units_dev, size_t units_bytes, int32_t B,
                    int32_t topk, void* ws_dev, size_t ws_bytes, void* out_dev, size_t out_bytes,
                    void* stream);

/* The whole step of a batch in one launch: the kernel also quantizes x and routes the
 * batch itself.  B <= 8: the experts page's capacity <= 8 path of ExpertsKernel, which
 * skips the plan and group kernels (one unit per distinct expert, its tokens in token
 * order, the same table moe_group writes for such a batch).  B > 8: the grouped kernel
 * (as moe_experts_run with col_tiles 0) with the plan and the chunk table made inside the
 * launch (experts page, plan_chunk and ExpertsGroupKernel; the early group release the
 * runtime page describes taken to its end): every workgroup quantizes a share of x and
 * publishes it (device-coherent stores, call-tagged flag), builds the chunk table from ids
 * in its own LDS, and starts its weight stream at once; its first x reads wait for the
 * whole plan.  The rows are the same bit for bit as moe_plan_group + moe_experts_run's;
 * options as there (col_tiles 0 or 2, grid, hidden dump), plus plan_dev and status_dev;
 * exchange, fc2_claims and ahead must be 0 (MOE_EINVAL), and batches beyond the grouped
 * kernel's limits (I > 384, more than 1024 chunks, more than 32 FC1 blocks or 8 FC2
 * chunks per workgroup, B * topk >= 65535) are MOE_EINVAL.
 * Inputs x_dev BF16 [B, D] and ids_dev i32 [B, topk]; outputs as moe_experts_run
 * (out_dev BF16 [B*topk, D], top-k order; optional hidden dump), plus the optional plan
 * and status word of moe_run_opts_t.  The FC1 -> FC2 exchange is chosen by
 * opts->exchange: by default (0) each hidden block's FC1 runs over the whole of K in one
 * workgroup, which publishes the finished block as call-tagged words; 1 and 2 are the
 * split-block variants of the experts kernel (the workspace from moe_workspace_bytes
 * holds any of them).  The FP32 sums of one call are summed in a fixed order, so repeated
 * calls give identical rows.  Ids out of range are skipped and flagged (status bit 0).
 * Errors: MOE_EINVAL for the cases of moe_experts_run; MOE_ENOSPACE likewise.
 * The same residency and no-overlap rules as moe_experts_run apply. */
int moe_decode_run(const moe_weights_t* weights, const moe_run_opts_t* opts, const void* x_dev,
                   const int32_t* ids_dev, int32_t B, int32_t topk, void* ws_dev, size_t ws_bytes,
                   void* out_dev, size_t out_bytes, void* stream);

/* moe_decode_run for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same step, the same
 * kernel and the same rows bit for bit, with no workspace argument.  What moe_decode_run
 * keeps in the workspace (the call counters, the default status word and the call-tagged
 * hidden exchange) lives in a fixed scratch inside the library: one copy per device,
 * 1,188,096 bytes, zero when the library's code is loaded on that device and held until
 * the process ends.  The first call on a device looks up that device's copy
 * (hipGetSymbolAddress); no call allocates, frees or clears memory.
 * Limits (MOE_ELIMIT beyond them): the whole-K decode form only -- B <= 8, at most 128
 * distinct experts in the batch, B*topk <= 640, B*D/32 <= 2560, I <= 512; opts->exchange
 * must be 0.  Other arguments, options and errors as moe_decode_run.
 * All calls on one device share its scratch: calls that overlap in time on one device
 * (different streams without ordering, or several host threads) race and give wrong
 * rows; order them on one stream.  Calls on different devices are independent. */
int moe_decode_run_noalloc(const moe_weights_t* weights, const moe_run_opts_t* opts, const void* x_dev,
                           const int32_t* ids_dev, int32_t B, int32_t topk, void* out_dev, size_t out_bytes,
                           void* stream);

/* ------------------------------------------------------------- combine ---- */

/* Weighted top-k combine of the output rows (experts page, ExpertsKernel.finalize, the
 * arithmetic without the cross-rank multicast):
 *     out[t, d] = sum over s < topk of weights[t, s] * rows[t*topk + s, d]
 * accumulated in FP32 with fused multiply-adds in slot order s = 0, 1, ..., rounded
 * once to BF16 (round to nearest even).
 *   rows_dev    BF16 [B*topk, D], as written by moe_experts_run (rows_bytes >= B*topk*D*2)
 *   weights_dev FP32 [B, topk], the routing weights in the caller's top-k order
 *   out_dev     BF16 [B, D] (out_bytes >= B*D*2); must not overlap rows_dev
 * D must be a multiple of 8.  Returns MOE_EINVAL / MOE_ENOSPACE as the other calls. */
int moe_combine(const void* rows_dev, size_t rows_bytes, const float* weights_dev, int32_t B, int32_t topk,
                int32_t D, void* out_dev, size_t out_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MX_H */
