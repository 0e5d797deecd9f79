/* fc.h -- C ABI of libfc.so: one GPU's share of a "flash all-reduce" on MI355X (gfx950).
 *
 * The operations follow three descriptions of tensor-parallel all-reduce for LLM inference:
 *  - Flash Communication: Reducing Tensor Parallelization Bottleneck for Fast Large Language Model
 *    Inference (abstract; summary "Core ideas of the solution"): low-bit fine-grained quantization of
 *    activations, and a two-step all-reduce (reduce-scatter, then all-gather).
 *  - flash-comm (abstract): self-synchronizing transfers, each data block carrying evidence of its
 *    readiness that the receiver validates without a barrier; reduction order decoupled from
 *    transport order.
 *  - TokenWeave: Efficient Compute-Communication Overlap for Distributed LLM Inference (abstract):
 *    fused AllReduce-RMSNorm on few compute units, overlapped with the other half-batch's compute.
 * The pages fix no bit widths, layouts or formulas; the choices made here are stated per call.
 *
 * Conventions for every call
 *  - Pointers are DEVICE pointers unless marked [host].  The caller owns all memory and keeps it alive
 *    until the enqueued work has finished.  No call allocates, frees or synchronizes.
 *  - Each call validates its arguments on the host before touching the GPU, then enqueues its kernel(s)
 *    on `stream` (0 = the null stream) and returns.  Device faults are asynchronous and surface at the
 *    caller's next synchronization.
 *  - Status codes: FC_E_NULL a required pointer is NULL; FC_E_ARG a value outside the supported set
 *    (bits not 4/8, group not 32/64/128/256, R not in [1,16], eps not > 0, block_slots not
 *    32/64/128/256, an input range that partially overlaps an output range); FC_E_SHAPE sizes that do
 *    not divide (n % group, L % group, n % hidden, hidden % 8, n % (2*block_slots)) or exceed the
 *    limits below; FC_E_ALIGN a data pointer not 16-byte aligned (meta: 4-byte); FC_E_LAUNCH the HIP
 *    launch failed (the hipError_t is kept for fc_last_hip_error()).
 *  - Out-of-contract values (NaN, Inf, |x| > 65504, group ranges or sums outside the fp16 range) give
 *    unspecified results but never an out-of-bounds access.
 *  - bf16 and fp16 values are passed as their uint16_t bit patterns.
 *  - Element counts are limited to 2^31 - 16 per rank buffer (n, L, rows*hidden).
 */
#ifndef FC_H
#define FC_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FC_ABI_VERSION 5

typedef enum {
    FC_OK = 0,
    FC_E_NULL = 1,
    FC_E_ARG = 2,
    FC_E_SHAPE = 3,
    FC_E_ALIGN = 4,
    FC_E_LAUNCH = 5
} fc_status;

/* One quantized message of n elements in flat groups of `group` consecutive elements.
 *  codes: n*bits/8 bytes.  bits = 8: byte i holds code i.  bits = 4: byte i holds code 2i in its low
 *         nibble and code 2i+1 in its high nibble.  Codes are unsigned, 0 .. 2^bits - 1.
 *  meta:  n/group words; bits 0..15 = fp16 scale s, bits 16..31 = fp16 zero-point z of the group.
 *  Value of code q: fl(q*s + z) in fp32 (q*s is exact, so this is one rounding).
 *  Quantizer (asymmetric min/max): z = largest fp16 <= min(x) (a -0 minimum counts as +0);
 *  s = smallest fp16 >= fp32((max(x) - z) / (2^bits - 1)), or +0 when max(x) == z;
 *  q = round-half-even((x - z) * fp32(1/s)) clamped to [0, 2^bits - 1] (all codes 0 when s == 0). */
typedef struct {
    uint8_t* codes;
    uint32_t* meta;
} fc_qmsg;

/* Fused residual-add + RMSNorm epilogue (TokenWeave, abstract), per row of `hidden` elements of the
 * fp32 all-reduced value y:
 *   h = y + residual (fp32);  residual_out = bf16(h);  r = 1/sqrt(mean(h*h) + eps);
 *   out = bf16((h * r) * gamma).  bf16 rounding is to nearest even. */
typedef struct {
    const uint16_t* residual;  /* bf16 [rows*hidden], or NULL for no residual add */
    const uint16_t* gamma;     /* bf16 [hidden], required */
    float eps;                 /* > 0 */
    int64_t hidden;            /* row length H: a multiple of 8, at most 65536 */
    uint16_t* out;             /* bf16 [rows*hidden], required */
    uint16_t* residual_out;    /* bf16 [rows*hidden] or NULL; may be exactly `residual` (in place) */
} fc_norm;

/* Group-quantize n bf16 values (Flash Communication: low-bit fine-grained activation quantization).
 * x: bf16 [n], 16-byte aligned; n % group == 0.  Several ranks' buffers laid end to end may be
 * quantized in one call (their boundaries fall on group boundaries).  out.codes: n*bits/8 bytes,
 * out.meta: n/group words. */
fc_status fc_quantize(const uint16_t* x, int64_t n, int bits, int group, fc_qmsg out, hipStream_t stream);

/* Reduce-scatter receive side (Flash Communication, two-step all-reduce, step one; flash-comm: fixed
 * reduction order).  For each of n_shards shards, in[shard*R + r] [host array] is rank r's quantized
 * chunk of that shard (L elements, bits_in, `group`).  Each element is dequantized from every rank and
 * summed in fp32 as a left fold in ascending rank order (rank 0 first), whatever order the chunks
 * arrived in; the fp32 sum is requantized at bits_out into out[shard] [host array] (L elements), the
 * payload of the all-gather step.  L % group == 0.  Several launches are enqueued when n_shards * R
 * exceeds 128. */
fc_status fc_reduce_shard(const fc_qmsg* in, int R, int64_t L, int n_shards, int bits_in, int bits_out,
                          int group, const fc_qmsg* out, hipStream_t stream);

/* Reduce-scatter receive side with the norm before the all-gather (TokenWeave, abstract: the RMSNorm
 * fused with the all-reduce and moved relative to the communication, so each rank normalizes only its
 * 1/R of the rows).  in, R, L, n_shards, bits_in, group as for fc_reduce_shard; every shard holds whole
 * rows: L % norm->hidden == 0 and norm->hidden % group == 0.  For each shard: S = the fixed-order fp32
 * fold of the R dequantized chunks; h = S + residual; residual_out = bf16(h); the rows of h are
 * normalized in fp32, o = (h * (1/sqrt(sum(h^2)/hidden + eps))) * gamma, and o is quantized at bits_out
 * into out[shard] (the all-gather payload; fc_gather_dequant with y gives the normalized bf16 rows).
 * The sum of squares has a fixed order, because o decides integer codes: per 8-element chunk a left
 * fold of h*h, then a pairwise tree over the chunks of the row (the chunk count padded to a power of
 * two with zeros).  norm->residual and norm->residual_out (bf16 [n_shards*L], shard i's rows at i*L;
 * either may be NULL; they may alias exactly) and norm->gamma, eps, hidden as for the other epilogues;
 * norm->out must be NULL (FC_E_ARG otherwise).  Outputs may not overlap inputs or each other. */
fc_status fc_reduce_shard_norm(const fc_qmsg* in, int R, int64_t L, int n_shards, int bits_in, int bits_out,
                               int group, const fc_norm* norm, const fc_qmsg* out, hipStream_t stream);

/* All-gather receive side (Flash Communication, two-step all-reduce, step two).  shards[s] [host array,
 * R entries] holds elements [s*L, (s+1)*L) of the flat [rows, hidden] result.  Each element is
 * dequantized to fp32.  y (bf16 [R*L], or NULL) receives bf16(value).  norm (or NULL) applies the
 * residual-add + RMSNorm epilogue to the fp32 values, rows = R*L/hidden.  y and norm may not both be
 * NULL. */
fc_status fc_gather_dequant(const fc_qmsg* shards, int R, int64_t L, int bits, int group, uint16_t* y,
                            const fc_norm* norm, hipStream_t stream);

/* Unquantized fused all-reduce + residual-add + RMSNorm (TokenWeave, abstract).  parts [host array, R
 * entries]: bf16 [rows*hidden] partial sums.  y = fp32 left fold over ranks in ascending order, then the
 * epilogue of `norm` (required).  max_workgroups bounds the number of workgroups (the compute-unit
 * footprint); 0 = one workgroup per row.  Rows are independent, so any split of the rows into
 * separate calls gives the same bits. */
fc_status fc_reduce_rmsnorm(const uint16_t* const* parts, int R, int64_t rows, const fc_norm* norm,
                            int max_workgroups, hipStream_t stream);

/* Receiver counters (fc_ll_unpack_reduce, fc_ll_gather, fc_ll_poll_unpack_reduce, fc_flag_unpack_reduce).
 * A counters buffer is FC_COUNTER_WORDS uint32 words, 8-byte aligned, zeroed by the caller (the calls
 * add to it): FC_COUNTER_GROUPS groups of counter words, group g starting at word g * FC_COUNTER_STRIDE.  A workgroup of a receiver adds its counts to group (its index mod
 * FC_COUNTER_GROUPS); the total of count k is the sum of word k over the groups.  Device-scope atomics
 * on one address complete one at a time, and a receiver's workgroups all count at about the same time,
 * at the end: spread over eight addresses 512 bytes apart they no longer queue on one (8-rank slot
 * receiver, pass 1: 10.0 -> 8.2 us).  counters may be NULL: nothing is counted and no atomic is issued
 * (the stale and done flags hold every verdict). */
#define FC_COUNTER_GROUPS 8
#define FC_COUNTER_STRIDE 128
#define FC_COUNTER_WORDS (FC_COUNTER_GROUPS * FC_COUNTER_STRIDE)

/* Epochs (every call below that takes one): the readiness evidence is a comparison with `epoch` and
 * nothing else, so a buffer must not already hold the epoch of a message it has not yet received: a
 * caller uses a new epoch for each message through the same buffers, never one that an earlier message
 * or the buffers' initial contents carry (zero-filled buffers: start at 1).  The library cannot tell a
 * reused epoch from a delivered message.
 *
 * Self-synchronizing receive side (flash-comm, abstract).  slots [host array, R entries]: uint64 [n/2]
 * per rank; slot k = bf16 element 2k (bits 0..15), element 2k+1 (bits 16..31), epoch word (bits
 * 32..63).  A block is `block_slots` consecutive slots; nblk = n/2/block_slots.  For each block b with
 * done[b] == 0: stale[r*nblk + b] = 1 if any slot of rank r's copy carries an epoch word != epoch, else
 * 0; if no rank is stale the block is reduced (fp32 left fold in ascending rank order, bf16 out) and
 * done[b] = 1, otherwise out is left untouched and the block is pending.  Blocks with done[b] != 0 are
 * skipped: nothing of theirs is written (their slots may still be read).  counters (FC_COUNTER_WORDS,
 * grouped as above, or NULL): count 0 += stale (rank, block) pairs seen, count 1 += pending blocks, in
 * one 64-bit atomic add per workgroup; count 0 must not wrap (a call adds at most R*nblk < 2^29).
 * Calling again after late blocks have been rewritten completes them with the same bits as if they had
 * been on time.  n % (2*block_slots) == 0. */
fc_status fc_ll_unpack_reduce(const uint64_t* const* slots, int R, int64_t n, int block_slots, uint32_t epoch,
                              uint16_t* out, uint8_t* stale, uint8_t* done, uint32_t* counters,
                              hipStream_t stream);

/* Standalone all-gather on self-synchronizing blocks (flash-comm, abstract: every block carries evidence
 * of its readiness; the same mechanism serves an all-gather).  slots [host array, R entries]: rank r's
 * uint64 [nwords] slots, payload word k in bits 0..31 of slot k (bf16 pairs, or the words of a quantized
 * message: codes, then meta, in one buffer), epoch word in bits 32..63.  A block is `block_slots`
 * consecutive slots; nblk = nwords / block_slots.  For each (rank r, block b) with done[r*nblk + b] == 0:
 * stale[r*nblk + b] = 1 if any slot carries an epoch word != epoch, else 0; a valid block's words are
 * copied to out[r] (uint32 [nwords], host array of R device pointers, 8-byte aligned) and done is set; a
 * stale one is left untouched and pending.  counters (FC_COUNTER_WORDS, grouped as above, or NULL):
 * count 0 += stale (rank, block) pairs and count 1 += pending pairs (the same pairs: nothing is reduced
 * across ranks), in one 64-bit atomic add per workgroup.  A done block's slots may still be read.
 * Calling again after late blocks have been rewritten completes them.  nwords % block_slots == 0. */
fc_status fc_ll_gather(const uint64_t* const* slots, int R, int64_t nwords, int block_slots, uint32_t epoch,
                       uint32_t* const* out, uint8_t* stale, uint8_t* done, uint32_t* counters, hipStream_t stream);

/* Sender side of the slots above, used to emulate R peers writing at the same time (one launch): packs
 * rank r's bf16 x[r] [n] into n/2 slots[r] tagged with `epoch`, writing blocks in the order
 * block_order[r][0..nblk) (an int32 permutation of the block indices; block_order NULL, or an entry NULL,
 * for ascending).  x, block_order, slots: host arrays of R device pointers.  Each slot is written with one
 * agent-scope atomic 64-bit store, so a receiver reading at the same time sees its payload and epoch word
 * together.  pace (0..65536): each wavefront of the packer first sleeps pace x 512 clocks (slow senders
 * for runs where the receiver starts first; 0 for none).  The result does not depend on the order or the
 * pace.  No rank's slots may overlap any rank's input or order, or another rank's slots. */
fc_status fc_ll_pack(const uint16_t* const* x, int R, int64_t n, int block_slots, uint32_t epoch,
                     const int32_t* const* block_order, int pace, uint64_t* const* slots, hipStream_t stream);

/* Receiver of the slots above that may run while the senders still write (flash-comm, abstract: the
 * receiver validates the blocks it needs itself, with no barrier between GPUs).  Arguments, verdicts and
 * outputs as for fc_ll_unpack_reduce, except: every slot is read with an agent-scope atomic 64-bit load;
 * a wavefront owns tiles of 256 slots and, while a rank still has a stale block in the tile, re-reads
 * that rank's slots of the tile after a short sleep, at most max_polls times (0..2^20; 0 = one look, with
 * the results of fc_ll_unpack_reduce); the verdicts are those of the last look.  max_workgroups > 0 caps
 * the grid (the tiles are then walked with a stride), leaving compute units to a sender running at the
 * same time; 0 = one tile per wavefront.  counters (FC_COUNTER_WORDS, grouped as above, or NULL):
 * count 0 stale (rank, block) pairs and count 1 pending blocks at the last look (one 64-bit atomic add
 * per workgroup), count 2 += re-reads summed over wavefronts, count 3 unused.  The call always ends: a
 * block still stale after the budget is left pending for a later call. */
fc_status fc_ll_poll_unpack_reduce(const uint64_t* const* slots, int R, int64_t n, int block_slots, uint32_t epoch,
                                   int max_polls, int max_workgroups, uint16_t* out, uint8_t* stale, uint8_t* done,
                                   uint32_t* counters, hipStream_t stream);

/* Readiness by one flag word per block (flash-comm, abstract: the readiness encoding is a choice the
 * protocol selector makes; this one sends the payload unchanged, plus one word per block).  payload
 * [host array, R entries]: rank r's bf16 [n], 16-byte aligned; flags [host array, R entries]: rank r's
 * uint32 [nblk], 4-byte aligned; a block is block_elems consecutive elements (a power of two, 512 ..
 * 65536), nblk = n / block_elems.  The sender stores a block's payload, then the epoch into its flag
 * word with release order (fc_flag_pack).  For each block b with done[b] == 0: rank r's copy is stale
 * iff flags[r][b] != epoch, and stale[r*nblk + b] = 1, else 0; if no copy is stale, out (bf16 [n]) =
 * bf16 of the fp32 sum of the R copies folded in ascending rank order, and done[b] = 1; otherwise the
 * block stays pending and out is untouched.  The payload of a stale copy is never read.  Flags are read
 * with agent-scope atomic loads, re-read after a short sleep while a copy in the wavefront's tile (one
 * block, two of 512 elements) is stale, at most max_polls times (0..2^20; 0 = one look), then one
 * acquire fence precedes the payload loads.  max_workgroups and counters as for
 * fc_ll_poll_unpack_reduce.  Calling again after late blocks have been published completes them with
 * the same bits as if they had been on time. */
fc_status fc_flag_unpack_reduce(const uint16_t* const* payload, const uint32_t* const* flags, int R, int64_t n,
                                int block_elems, uint32_t epoch, int max_polls, int max_workgroups, uint16_t* out,
                                uint8_t* stale, uint8_t* done, uint32_t* counters, hipStream_t stream);

/* Sender side of the flag encoding, used to emulate R peers writing at the same time (one launch): writes
 * rank r's x[r] (bf16 [n]) into payload[r] in the block order block_order[r] (as for fc_ll_pack), and
 * publishes every block by storing epoch into flags[r][b] after a release fence.  A workgroup writes a
 * span of consecutive entries of the order (2^13 to 2^17 elements, growing with n; at least one block),
 * waits for its stores, meets at a barrier, fences once with release order at agent scope and stores
 * the span's flags: a receiver that reads a flag and then fences with acquire order sees the whole
 * block.  pace: sleeps of 512 clocks before each span (0..65536).  block_elems as for
 * fc_flag_unpack_reduce.  Host arrays of R device pointers; no output may overlap an input or another
 * output. */
fc_status fc_flag_pack(const uint16_t* const* x, int R, int64_t n, int block_elems, uint32_t epoch,
                       const int32_t* const* block_order, int pace, uint16_t* const* payload, uint32_t* const* flags,
                       hipStream_t stream);

/* Measurement helper: copies `bytes` (a multiple of 16, at most 2^40, 16-byte aligned pointers, no
 * overlap) with one non-temporal 16-byte load and store per lane; its bandwidth is the practical HBM
 * ceiling the kernels above are compared with. */
fc_status fc_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream);

/* Measurement helper: the HBM ceilings the kernels are compared with, by access mix.  mode 0: the copy
 * above (src -> dst, `bytes` each way); mode 1: read `bytes` of src (16-byte aligned) with one
 * non-temporal 16-byte load per lane (1024-lane workgroups), each lane folding its four words so the
 * load stays; dst is a 4-byte sink that receives 0x9E3779B9 only if some lane's fold equals that value;
 * mode 2: write `bytes` of dst with one 16-byte store per lane, uint4 i = (0x3F803F80, i mod 2^32, 0, 0)
 * (src unused, may be NULL).  bytes: a multiple of 16, at most 2^40. */
fc_status fc_bandwidth_probe(const void* src, void* dst, int64_t bytes, int mode, hipStream_t stream);

const char* fc_status_string(fc_status s);
int fc_last_hip_error(void); /* hipError_t of the last FC_E_LAUNCH on this thread */
int fc_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* FC_H */
