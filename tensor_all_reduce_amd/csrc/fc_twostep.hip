// fc_twostep.hip -- gfx950 kernels of the quantized two-step all-reduce and of the fused row epilogues
// (group quantization, fixed-order shard reduce, all-gather dequantize, residual-add + RMSNorm rows,
// unquantized reduce + RMSNorm, the norm before the all-gather) and their launchers.
//
// Layout rule for every kernel: one wavefront-wide memory instruction covers one contiguous span, lane i
// at base + i * width (16 bytes of bf16, 16, 8 or 4 bytes of codes), so each instruction
// moves whole cache lines.  A lane therefore holds 8 consecutive bf16 elements (or 16 codes) per
// instruction, and a quantization group spans G/8 (or G/16) aligned lanes whose min/max are combined
// with DPP.  One exception: the norm-before-gather reduce gives a lane 16 consecutive elements, so its
// codes stay contiguous per instruction and its residual takes two 16-byte accesses 32 bytes apart.
// Intermediate fp32 values stay in registers; RMSNorm row sums use DPP inside a wavefront and LDS across
// wavefronts.  Nothing here is a contraction, so matrix cores are not used.
#include <type_traits>

#include "fc_device.h"
#include "fc_launch.h"

namespace fc {

__device__ __forceinline__ void unpack_bf16x8(uint4 u, float (&v)[8]) {
    v[0] = bf16_lo(u.x);
    v[1] = bf16_hi(u.x);
    v[2] = bf16_lo(u.y);
    v[3] = bf16_hi(u.y);
    v[4] = bf16_lo(u.z);
    v[5] = bf16_hi(u.z);
    v[6] = bf16_lo(u.w);
    v[7] = bf16_hi(u.w);
}

__device__ __forceinline__ uint4 pack_bf16x8(const float (&v)[8]) {
    return make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                      pack_bf16x2(v[6], v[7]));
}

// Dequantize the 8 codes of one lane-chunk (8 bytes of 8-bit codes or 4 bytes of 4-bit codes).
template <int BITS>
__device__ __forceinline__ void dequant8(const void* p, float s, float z, float (&y)[8]) {
    if constexpr (BITS == 8) {
        const uint2 w = lds8(p);
        Unpack<8>::run(w.x, s, z, y);
        Unpack<8>::run(w.y, s, z, y + 4);
    } else {
        Unpack<4>::run(lds4(p), s, z, y);
    }
}

// =====================================================================================================
// Group quantization (Flash Communication, summary "Core ideas of the solution": low-bit fine-grained
// quantization of activations).  Lane-chunk = 8 bf16 (16 bytes); a group of G spans LPG = G/8 lanes.
// Each lane handles K lane-chunks ("slots"), 64 chunks apart, so a wavefront covers K * 64/LPG groups.
// Min/max are reduced per slot with DPP; then lane g*LPG + j picks slot j's values of its group g, so the
// per-group step (zero point, scale, reciprocal: mostly divisions) runs once for all K slots, and its
// results are broadcast back to the group's lanes.  K = 2 or 4 for large inputs (independent 16-byte
// loads in flight, per-group work shared), K = 1 for small, latency-bound ones.
// =====================================================================================================
template <int BITS, int G, int K>
__global__ __launch_bounds__(256) void k_quantize(const uint16_t* __restrict__ x, uint32_t nchunks,
                                                  uint8_t* __restrict__ codes, uint32_t* __restrict__ meta) {
    constexpr int LPG = G / 8;
    constexpr int CB = BITS;  // code bytes per 8-element chunk: 8 or 4
    static_assert(K == 1 || K == 2 || K == 4, "slot select below");
    static_assert(K <= LPG, "the K slots of a group are gathered into K of its lanes");
    const int lane = threadIdx.x & 63;
    const uint32_t wbase = (blockIdx.x * 4u + (threadIdx.x >> 6)) * (64u * K);  // < 2^31 (launcher)
    float v[K][8];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        // Chunks past the end: whole groups lie on either side of it, so these lanes recompute the last
        // chunk (keeping their DPP partners' data valid) and store nothing.
        const uint32_t c = min(wbase + 64u * k + lane, nchunks - 1u);
        unpack_bf16x8(lds16(x + (size_t)c * 8), v[k]);
    }
    float lo[K], hi[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        lane_minmax<8>(v[k], lo[k], hi[k]);
        lo[k] = group_min<LPG>(lo[k]);
        hi[k] = group_max<LPG>(hi[k]);
    }
    // lane g*LPG + j takes slot j % K of group g
    float sl = lo[0], sh = hi[0];
    if constexpr (K >= 2) {
        const bool b0 = lane & 1;
        sl = b0 ? lo[1] : lo[0];
        sh = b0 ? hi[1] : hi[0];
        if constexpr (K == 4) {
            const bool b1 = lane & 2;
            sl = b1 ? (b0 ? lo[3] : lo[2]) : sl;
            sh = b1 ? (b0 ? hi[3] : hi[2]) : sh;
        }
    }
    const GroupQ q = group_params<BITS>(sl, sh);
    {
        const int j = lane % LPG;
        const uint32_t c0 = wbase + 64u * (j % K) + (lane - j);  // first chunk of the group this lane holds
        if (j < K && c0 < nchunks) meta[c0 / LPG] = q.meta;
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
        float z = q.z, inv = q.inv;
        if constexpr (K > 1) {
            if (k == 0) { z = group_bcast<LPG, 0>(q.z, lane); inv = group_bcast<LPG, 0>(q.inv, lane); }
            if (k == 1) { z = group_bcast<LPG, 1>(q.z, lane); inv = group_bcast<LPG, 1>(q.inv, lane); }
            if constexpr (K == 4) {
                if (k == 2) { z = group_bcast<LPG, 2>(q.z, lane); inv = group_bcast<LPG, 2>(q.inv, lane); }
                if (k == 3) { z = group_bcast<LPG, 3>(q.z, lane); inv = group_bcast<LPG, 3>(q.inv, lane); }
            }
        }
        uint32_t w[BITS / 4];
        encode_lane<BITS, 8>(v[k], z, inv, w);
        const uint32_t c = wbase + 64u * k + lane;
        if (c < nchunks) {
            if constexpr (BITS == 8) stm8(codes + (size_t)c * CB, make_uint2(w[0], w[1]));
            else stm4(codes + (size_t)c * CB, w[0]);
        }
    }
}

template <int BITS, int K>
static void quantize_k(const QuantizeParams& p, int64_t nchunks, hipStream_t s) {
    // Pieces of at most 2^30 chunks keep every in-kernel chunk index below 2^31; a piece is a whole
    // number of groups, so it starts on a group boundary.
    constexpr int64_t PIECE = (int64_t)1 << 30;
    for (int64_t c0 = 0; c0 < nchunks; c0 += PIECE) {
        const uint32_t nc = (uint32_t)(nchunks - c0 < PIECE ? nchunks - c0 : PIECE);
        const dim3 grid((nc + 256u * K - 1) / (256u * K));
        const uint16_t* x = p.x + c0 * 8;
        uint8_t* codes = p.codes + c0 * BITS;
        uint32_t* meta = p.meta + c0 * 8 / p.group;
        switch (p.group) {
            case 32: k_quantize<BITS, 32, K><<<grid, 256, 0, s>>>(x, nc, codes, meta); break;
            case 64: k_quantize<BITS, 64, K><<<grid, 256, 0, s>>>(x, nc, codes, meta); break;
            case 128: k_quantize<BITS, 128, K><<<grid, 256, 0, s>>>(x, nc, codes, meta); break;
            default: k_quantize<BITS, 256, K><<<grid, 256, 0, s>>>(x, nc, codes, meta); break;
        }
    }
}

template <int BITS>
static hipError_t quantize_bits(const QuantizeParams& p, hipStream_t s) {
    const int64_t nchunks = p.n / 8;
    // below ~4096 workgroups of K = 4 the launch cannot fill the chip's 256 compute units several times;
    // above, 4-bit codes run best with K = 2 and 8-bit codes with K = 4 (measured on the 70B prefill batch)
    if (nchunks >= (int64_t)4096 * 1024) quantize_k<BITS, BITS == 4 ? 2 : 4>(p, nchunks, s);
    else quantize_k<BITS, 1>(p, nchunks, s);
    return hipGetLastError();
}

hipError_t launch_quantize(const QuantizeParams& p, hipStream_t s) {
    return p.bits == 8 ? quantize_bits<8>(p, s) : quantize_bits<4>(p, s);
}

// =====================================================================================================
// Reduce-scatter receive side (two-step all-reduce, step one).  Block row y = shard; lane-chunk = E
// elements (16: 16 or 8 bytes of codes per rank; 8 or 4 for small shards, more lanes in flight);
// a group spans G/E lanes.  Each lane dequantizes its chunk from every rank's message and folds the
// values in fp32 in ascending rank order (flash-comm: reduction order fixed, independent of arrival
// order), then requantizes the fp32 sums for the all-gather step.
// =====================================================================================================
constexpr int kReduceShards = kMaxReduceIn / kMaxRanks;  // shards per launch
struct ReduceKArgs {
    // [shard in launch][rank]: rank r's chunk of the shard.  Entries r >= R repeat rank R-1, so a table
    // address depends only on the block index and every pointer arrives in one kernel-argument fetch.
    const uint8_t* in_codes[kReduceShards][kMaxRanks];
    const uint32_t* in_meta[kReduceShards][kMaxRanks];
    uint8_t* out_codes[kReduceShards];
    uint32_t* out_meta[kReduceShards];
};

// E codes of B bits: load (E*B/8 bytes) as 32-bit words
template <int E, int B>
__device__ __forceinline__ void load_codes(const uint8_t* p, uint32_t (&w)[E * B / 32]) {
    if constexpr (E * B / 8 == 16) {
        const uint4 u = lds16(p);
        w[0] = u.x;
        w[1] = u.y;
        w[2] = u.z;
        w[3] = u.w;
    } else if constexpr (E * B / 8 == 8) {
        const uint2 u = lds8(p);
        w[0] = u.x;
        w[1] = u.y;
    } else {
        w[0] = lds4(p);
    }
}

template <int E, int B>
__device__ __forceinline__ void store_codes(uint8_t* p, const uint32_t (&w)[E * B / 32]) {
    if constexpr (E * B / 8 == 16) stm16(p, make_uint4(w[0], w[1], w[2], w[3]));
    else if constexpr (E * B / 8 == 8) stm8(p, make_uint2(w[0], w[1]));
    else stm4(p, w[0]);
}

// R8: the rank count is 8 (every workload here), known at compile time.  Otherwise the compiler, not
// knowing which ranks are folded, moves one rank's loads into its conditional fold, behind the scalar load
// of its pointer, and that rank's data arrives a memory round trip late.
template <int B1, int B2, int G, int E, bool R8>
__global__ __launch_bounds__(256) void k_reduce(const int64_t nchunks, const int R_arg, const ReduceKArgs a) {
    constexpr int LPG = G / E;
    constexpr int IN_W = E * B1 / 32;  // input code words per rank
    constexpr int RB = 8;              // ranks loaded per batch
    const int R = R8 ? 8 : R_arg;
    __builtin_assume(R >= 1);  // validated on the host: rank 0 is always folded
    const int shard = blockIdx.y;
    const int64_t c0 = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const bool valid = c0 < nchunks;
    const int64_t c = valid ? c0 : nchunks - 1;  // whole groups lie on either side of the end
    const int64_t gidx = c / LPG;
    // 32-bit byte offsets from each rank's (wavefront-uniform) chunk base: a shard's codes are at most
    // 2^31 bytes, and a uniform base plus a 32-bit lane offset needs no 64-bit address arithmetic per rank
    const uint32_t coff = (uint32_t)c * (uint32_t)(E * B1 / 8);
    const uint32_t moff = (uint32_t)gidx * 4u;
    float acc[E];
    // All RB loads of a batch are issued unconditionally (ranks past R re-read rank R-1 and are ignored),
    // so no branch separates them and they are all in flight together.  The first batch is outside the
    // loop: its loads wait for nothing but the kernel arguments (not for R).
    uint32_t wv[RB][IN_W];
    uint32_t mv[RB];
    auto load_batch = [&](int r0) {
#pragma unroll
        for (int j = 0; j < RB; ++j) {
            load_codes<E, B1>(a.in_codes[shard][r0 + j] + coff, wv[j]);
            mv[j] = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(a.in_meta[shard][r0 + j]) + moff);
        }
    };
    auto fold_batch = [&](int r0) {
#pragma unroll
        for (int j = 0; j < RB; ++j) {
            if (r0 + j < R) {  // uniform
                const float sc = meta_scale(mv[j]);
                const float z = meta_zero(mv[j]);
                float d[E];
#pragma unroll
                for (int k = 0; k < IN_W; ++k) Unpack<B1>::run(wv[j][k], sc, z, d + k * Unpack<B1>::PER_WORD);
                if (r0 + j == 0) {
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[e] = d[e];
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[e] = acc[e] + d[e];
                }
            }
        }
    };
    // Small launches read the output pointers with the input tables, ahead of the loads (the empty asm pins
    // them there): left to itself the compiler reads them from the kernel arguments after the
    // requantization, a scalar round trip in front of the stores (decode shards 2.54 -> 2.45 us).  With
    // 16-element chunks (many resident workgroups) the late read is hidden, and pinning it measured slower.
    uint8_t* const oc = a.out_codes[shard];
    uint32_t* const om = a.out_meta[shard];
    load_batch(0);
    if constexpr (E < 16) asm volatile("" ::"s"(oc), "s"(om));
    // Every load of the batch is issued before the first fold: left to itself, the scheduler moves some
    // ranks' loads behind the first ranks' folds, and those ranks arrive a memory round trip late.
    __builtin_amdgcn_sched_barrier(0);
    fold_batch(0);
    for (int r0 = RB; r0 < R; r0 += RB) {  // more than 8 ranks
        load_batch(r0);
        __builtin_amdgcn_sched_barrier(0);
        fold_batch(r0);
    }
    uint32_t w[E * B2 / 32];
    uint32_t m;
    quantize_lane<B2, E, LPG>(acc, w, m);
    if (valid) {
        store_codes<E, B2>(oc + c * (E * B2 / 8), w);
        if ((threadIdx.x % LPG) == 0) om[gidx] = m;
    }
}

template <int B1, int B2, int E, bool R8>
static void reduce_launch_gr(int64_t nchunks, int R, const ReduceKArgs& a, int group, dim3 grid, hipStream_t s) {
    switch (group) {
        case 32: k_reduce<B1, B2, 32, E, R8><<<grid, 256, 0, s>>>(nchunks, R, a); break;
        case 64: k_reduce<B1, B2, 64, E, R8><<<grid, 256, 0, s>>>(nchunks, R, a); break;
        case 128: k_reduce<B1, B2, 128, E, R8><<<grid, 256, 0, s>>>(nchunks, R, a); break;
        default:
            if constexpr (E >= 8) k_reduce<B1, B2, 256, E, R8><<<grid, 256, 0, s>>>(nchunks, R, a);  // 4-element chunks: G <= 128
            break;
    }
}

template <int B1, int B2, int E>
static void reduce_launch_g(int64_t nchunks, int R, const ReduceKArgs& a, int group, dim3 grid, hipStream_t s) {
    if (R == 8) reduce_launch_gr<B1, B2, E, true>(nchunks, R, a, group, grid, s);
    else reduce_launch_gr<B1, B2, E, false>(nchunks, R, a, group, grid, s);
}

template <int E>
static hipError_t launch_reduce_e(const ReduceParams& p, hipStream_t s) {
    const int64_t nchunks = p.L / E;
    for (int s0 = 0; s0 < p.n_shards; s0 += kReduceShards) {
        const int ns = (p.n_shards - s0) < kReduceShards ? (p.n_shards - s0) : kReduceShards;
        ReduceKArgs a;
        for (int i = 0; i < ns; ++i) {
            for (int r = 0; r < kMaxRanks; ++r) {
                const int t = (s0 + i) * p.R + (r < p.R ? r : p.R - 1);
                a.in_codes[i][r] = p.in_codes[t];
                a.in_meta[i][r] = p.in_meta[t];
            }
        }
        for (int i = 0; i < ns; ++i) {
            a.out_codes[i] = p.out_codes[s0 + i];
            a.out_meta[i] = p.out_meta[s0 + i];
        }
        const dim3 grid((unsigned)((nchunks + 255) / 256), (unsigned)ns);
        const int R = p.R;
        if constexpr (E == 4) {
            reduce_launch_g<8, 8, 4>(nchunks, R, a, p.group, grid, s);  // chosen only for 8-bit codes and G <= 128
        } else {
            if (p.bits_in == 8 && p.bits_out == 8) reduce_launch_g<8, 8, E>(nchunks, R, a, p.group, grid, s);
            else if (p.bits_in == 4 && p.bits_out == 8) reduce_launch_g<4, 8, E>(nchunks, R, a, p.group, grid, s);
            else if (p.bits_in == 8 && p.bits_out == 4) reduce_launch_g<8, 4, E>(nchunks, R, a, p.group, grid, s);
            else reduce_launch_g<4, 4, E>(nchunks, R, a, p.group, grid, s);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_reduce(const ReduceParams& p, hipStream_t s) {
    // 16-element chunks need at least 8 workgroups (32 wavefronts) per compute unit of the 256 to keep
    // loads in flight; below that, halve the chunk (one GPU's prefill shard, 1024 workgroups of 16:
    // 7.4 -> 7.05 us with 2048 of 8).  Below 512 workgroups of 8-element chunks, 8-bit codes in and out
    // halve it again (4 bytes of codes per lane and rank; a group of up to 128 then spans at most 32 lanes).
    const int64_t wgs16 = (p.L / 16 + 255) / 256 * p.n_shards;
    const int64_t wgs8 = (p.L / 8 + 255) / 256 * p.n_shards;
    if (wgs8 < 512 && p.bits_in == 8 && p.bits_out == 8 && p.group <= 128) return launch_reduce_e<4>(p, s);
    return wgs16 < 2048 ? launch_reduce_e<8>(p, s) : launch_reduce_e<16>(p, s);
}

// =====================================================================================================
// All-gather receive side, plain mode: dequantize every shard to bf16.  Block row y = shard;
// lane-chunk = 8 elements (codes 8 or 4 bytes in, 16 bytes of bf16 out).
// =====================================================================================================
struct GatherKArgs {
    const uint8_t* codes[kMaxRanks];
    const uint32_t* meta[kMaxRanks];
    int64_t L;
    int64_t nchunks;  // 8-element chunks per shard
    int log2g;
    uint16_t* y;
};

template <int BITS>
__global__ __launch_bounds__(256) void k_gather_plain(const GatherKArgs a) {
    const int shard = blockIdx.y;
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= a.nchunks) return;
    const uint32_t m = a.meta[shard][(c * 8) >> a.log2g];
    float d[8];
    dequant8<BITS>(a.codes[shard] + c * BITS, meta_scale(m), meta_zero(m), d);
    sts16(a.y + shard * a.L + c * 8, pack_bf16x8(d));
}

// =====================================================================================================
// Row kernels: produce the fp32 all-reduced value y of one row, 8 elements (one lane-chunk) at a time,
// then apply the residual-add + RMSNorm epilogue (TokenWeave, abstract: fused AllReduce-RMSNorm).  A
// workgroup owns a row at a time and keeps h in registers (CPT chunks per lane, chunk j of a row at
// lane j % BT); sum(h^2) is reduced with DPP inside each wavefront and LDS across wavefronts.  Rows are
// walked with a stride of the grid size, so the grid (the compute-unit footprint) can be capped.
// =====================================================================================================
struct NormKArgs {
    const uint16_t* residual;
    const uint16_t* gamma;
    float eps;
    int hidden;
    uint16_t* out;
    uint16_t* residual_out;
};

// y from the R requantized shards of the all-gather step.  UNIFORM: every row lies inside one shard
// (L % H == 0), so the row's shard is the same for the whole workgroup and its message pointers are read
// straight from the kernel arguments; otherwise a chunk's shard is found per lane through a pointer
// table staged in LDS (which costs a barrier before the first load).
template <int BITS, bool UNIFORM>
struct GatherProducer {
    // the leading kernel arguments a0 = L (shard length), a1 = log2(group)
    const uint8_t* codes[kMaxRanks];
    const uint32_t* meta[kMaxRanks];

    static constexpr bool kNeedsSync = !UNIFORM;
    static constexpr int kOutBits = 0;  // bf16 output rows
    struct Shared {
        const uint8_t* codes[kMaxRanks];
        const uint32_t* meta[kMaxRanks];
    };
    struct Row {
        const uint8_t* codes;
        const uint32_t* meta;
        uint32_t base;  // flat index of the shard's first element
    };
    __device__ void init(Shared& sh) const {
        if constexpr (!UNIFORM) {
            if (threadIdx.x == 0) {
#pragma unroll
                for (int k = 0; k < kMaxRanks; ++k) {
                    sh.codes[k] = codes[k];
                    sh.meta[k] = meta[k];
                }
            }
        }
    }
    __device__ __forceinline__ Row begin_row(uint32_t rbase, uint32_t L, int) const {
        if constexpr (UNIFORM) {
            const uint32_t s = rbase / L;
            return Row{codes[s], meta[s], s * L};
        } else {
            return Row{nullptr, nullptr, 0};
        }
    }
    struct Raw {
        uint2 codes;  // 8 codes: 8 bytes (8-bit) or the low word (4-bit)
        uint32_t meta;
    };
    // Issue the loads of chunk i (no waiting); decode() turns them into y once they have arrived.
    __device__ __forceinline__ void fetch(const Shared& sh, const Row& row, uint32_t i, Raw& raw, uint32_t L,
                                          int log2g) const {
        const uint8_t* cp;
        const uint32_t* mp;
        uint32_t off;
        if constexpr (UNIFORM) {
            cp = row.codes;
            mp = row.meta;
            off = i - row.base;
        } else {
            const uint32_t s = i / L;  // an 8-element chunk never straddles a shard (L % 32 == 0)
            cp = sh.codes[s];
            mp = sh.meta[s];
            off = i - s * L;
        }
        raw.meta = *reinterpret_cast<const uint32_t*>(at(mp, (off >> log2g) << 2));
        if constexpr (BITS == 8) raw.codes = lds8(at(cp, off));
        else raw.codes = make_uint2(lds4(at(cp, off / 2)), 0u);
    }
    __device__ __forceinline__ void decode(const Raw& raw, float (&y)[8], const Row&, uint32_t, uint32_t, int) const {
        const float sc = meta_scale(raw.meta), z = meta_zero(raw.meta);
        if constexpr (BITS == 8) {
            Unpack<8>::run(raw.codes.x, sc, z, y);
            Unpack<8>::run(raw.codes.y, sc, z, y + 4);
        } else {
            Unpack<4>::run(raw.codes.x, sc, z, y);
        }
    }
};

// y from R bf16 partial sums, folded in fp32 in ascending rank order.
struct BF16ReduceProducer {
    // the leading kernel argument a0 = R; entries past R repeat rank R-1 (read and ignored), so the table
    // addresses need no kernel argument
    const uint16_t* parts[kMaxRanks];

    static constexpr bool kNeedsSync = false;
    static constexpr int kOutBits = 0;  // bf16 output rows
    struct Shared {};
    struct Row {};
    __device__ void init(Shared&) const {}
    __device__ __forceinline__ Row begin_row(uint32_t, uint32_t, int) const { return Row{}; }
    struct Raw {
        float y[8];
    };
    __device__ __forceinline__ void decode(const Raw& raw, float (&y)[8], const Row&, uint32_t, uint32_t, int) const {
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = raw.y[e];
    }
    __device__ __forceinline__ void fetch(const Shared&, const Row&, uint32_t i, Raw& raw, uint32_t R, int) const {
        float (&y)[8] = raw.y;
        constexpr int RB = 8;
        uint4 a[RB];
        auto fold = [&](int r0) {
#pragma unroll
            for (int j = 0; j < RB; ++j) {
                if (r0 + j < (int)R) {  // uniform
                    float v[8];
                    unpack_bf16x8(a[j], v);
                    if (r0 + j == 0) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) y[e] = v[e];
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e) y[e] = y[e] + v[e];
                    }
                }
            }
        };
        // first batch outside the loop: its loads wait for nothing but the kernel arguments
#pragma unroll
        for (int j = 0; j < RB; ++j) a[j] = lds16(at(parts[j], 2 * i));
        fold(0);
        for (int r0 = RB; r0 < (int)R; r0 += RB) {
#pragma unroll
            for (int j = 0; j < RB; ++j) a[j] = lds16(at(parts[r0 + j], 2 * i));
            fold(r0);
        }
    }
};

// y from the R quantized chunks of the row's shard (the reduce-scatter receive side), folded in fp32 in
// ascending rank order; the row's normalized values are quantized into the shard's all-gather message
// (the norm applied before the all-gather, TokenWeave, abstract).  Leading kernel arguments: a0 = L
// (shard length, a multiple of the row length), a1 = log2(group) | R << 8.  Pointer tables: [shard in
// launch][rank], entries past R repeat rank R-1.
constexpr int kNormShards = 8;  // shards per launch
template <int B1, int B2>
struct QReduceProducer {
    static constexpr bool kNeedsSync = false;
    static constexpr int kOutBits = B2;
    const uint8_t* codes[kNormShards][kMaxRanks];
    const uint32_t* meta[kNormShards][kMaxRanks];
    uint8_t* out_codes[kNormShards];
    uint32_t* out_meta[kNormShards];
    struct Shared {};
    struct Row {
        uint32_t s, base;  // shard in the launch, flat index of its first element
    };
    __device__ void init(Shared&) const {}
    __device__ __forceinline__ Row begin_row(uint32_t rbase, uint32_t L, int) const {
        const uint32_t s = rbase / L;
        return Row{s, s * L};
    }
    static constexpr int RB = 8;  // ranks whose loads are issued by fetch()
    struct Raw {
        uint32_t c[RB][B1 / 4];  // the chunk's 8 codes of rank j
        uint32_t m[RB];
    };
    __device__ __forceinline__ void load(const Row& row, uint32_t i, int r0, int log2g, Raw& raw) const {
        const uint32_t off = i - row.base;
#pragma unroll
        for (int j = 0; j < RB; ++j) {
            raw.m[j] = meta[row.s][r0 + j][off >> log2g];
            if constexpr (B1 == 8) {
                const uint2 u = lds8(codes[row.s][r0 + j] + off);
                raw.c[j][0] = u.x;
                raw.c[j][1] = u.y;
            } else {
                raw.c[j][0] = lds4(codes[row.s][r0 + j] + off / 2);
            }
        }
    }
    __device__ __forceinline__ void fetch(const Shared&, const Row& row, uint32_t i, Raw& raw, uint32_t, int a1) const {
        load(row, i, 0, a1 & 0xff, raw);
    }
    __device__ __forceinline__ void fold(const Raw& raw, int r0, int R, float (&y)[8]) const {
#pragma unroll
        for (int j = 0; j < RB; ++j) {
            if (r0 + j < R) {  // uniform
                float d[8];
#pragma unroll
                for (int w = 0; w < B1 / 4; ++w)
                    Unpack<B1>::run(raw.c[j][w], meta_scale(raw.m[j]), meta_zero(raw.m[j]), d + w * Unpack<B1>::PER_WORD);
                if (r0 + j == 0) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) y[e] = d[e];
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) y[e] = y[e] + d[e];
                }
            }
        }
    }
    __device__ __forceinline__ void decode(const Raw& raw, float (&y)[8], const Row& row, uint32_t i, uint32_t,
                                           int a1) const {
        const int R = a1 >> 8;
        fold(raw, 0, R, y);
        for (int r0 = RB; r0 < R; r0 += RB) {  // more than 8 ranks: the next batch is loaded here
            Raw more;
            load(row, i, r0, a1 & 0xff, more);
            fold(more, r0, R, y);
        }
    }
    // Quantize this lane's 8 normalized values (a group of G spans G/8 aligned lanes) and store them.
    template <int LPG>
    __device__ __forceinline__ void quantize_store(const Row& row, uint32_t i, const float (&o)[8], bool ok,
                                                   bool leader, int log2g) const {
        uint32_t w[B2 / 4];
        uint32_t m;
        quantize_lane<B2, 8, LPG>(o, w, m);
        if (ok) {
            const uint32_t off = i - row.base;
            if constexpr (B2 == 8) stm8(out_codes[row.s] + off, make_uint2(w[0], w[1]));
            else stm4(out_codes[row.s] + off / 2, w[0]);
            if (leader) out_meta[row.s][off >> log2g] = m;
        }
    }
    // t = the lane's index inside its row; groups never straddle a row end (hidden % group == 0).
    __device__ __forceinline__ void store(const Row& row, uint32_t i, const float (&o)[8], bool ok, int t,
                                          int a1) const {
        const int log2g = a1 & 0xff;
        switch (log2g) {  // uniform
            case 5: quantize_store<4>(row, i, o, ok, (t & 3) == 0, log2g); break;
            case 6: quantize_store<8>(row, i, o, ok, (t & 7) == 0, log2g); break;
            case 7: quantize_store<16>(row, i, o, ok, (t & 15) == 0, log2g); break;
            default: quantize_store<32>(row, i, o, ok, (t & 31) == 0, log2g); break;
        }
    }
};

// A workgroup of RPB * BT lanes keeps RPB rows in flight (sub-block j owns row base + j); RPB > 1 is used
// when the grid is capped well below the number of rows, so that each compute unit still has enough
// loads in flight.
// Scalars lead the argument list, so that they arrive preloaded in registers at dispatch (gfx950 kernel
// argument preloading); only the producer's pointer table is read from the argument segment.
template <class P, int BT, int CPT, int RPB>
__global__ __launch_bounds__(BT * RPB) void k_rows(const int64_t rows, const int hidden, const float eps,
                                                   const uint16_t* __restrict__ gamma,
                                                   const uint16_t* __restrict__ residual, uint16_t* out,
                                                   uint16_t* residual_out, const uint32_t a0, const int a1, const P p) {
    const NormKArgs na{residual, gamma, eps, hidden, out, residual_out};
    // Quantized output (the norm before the all-gather): the normalized values decide integer codes, so
    // the row's sum of squares follows a fixed order, the same for every launch shape: chunk partials
    // (left fold of h*h over the chunk's 8 elements), then a pairwise tree over the chunk index
    // c = t + k*BT, i.e. over the lane inside the wavefront (the DPP butterfly is that tree), over the
    // wavefronts, then over k.  bf16 output: any order (fused multiply-adds, lane-serial over k).
    constexpr bool kTreeSum = P::kOutBits != 0;
    __shared__ float s_part[RPB][kTreeSum ? CPT : 1][BT / 64];
    __shared__ typename P::Shared sh;
    p.init(sh);
    if constexpr (P::kNeedsSync) __syncthreads();
    const int H = na.hidden;
    const int nch = H >> 3;
    const int sub = RPB == 1 ? 0 : threadIdx.x / BT;  // row slot inside the workgroup
    const int t = threadIdx.x - sub * BT;       // lane inside the row
    const int lane = threadIdx.x & 63, wid = t >> 6;
    // Loads are never issued inside a lane-divergent branch (the compiler would wait for each one before
    // leaving the branch): lanes past the end of a row load a clamped, valid chunk and only their stores
    // and contributions are masked.
    // gamma does not depend on the row: load this lane's chunks once (for the longest rows, whose
    // registers are taken by h, reload it per row instead)
    constexpr bool kHoistGamma = CPT <= 4;
    uint4 g[kHoistGamma ? CPT : 1];  // kept as bf16 words until used, so that nothing waits for it early
    if constexpr (kHoistGamma) {
#pragma unroll
        for (int k = 0; k < CPT; ++k) g[k] = ld16(at(na.gamma, (uint32_t)min(t + k * BT, nch - 1) * 16));
    }
    for (int64_t row0 = (int64_t)blockIdx.x * RPB; row0 < rows; row0 += (int64_t)gridDim.x * RPB) {
        const int64_t row = row0 + sub;
        const bool has_row = row < rows;
        const uint32_t rbase = (uint32_t)((has_row ? row : rows - 1) * H);
        const typename P::Row pr = p.begin_row(rbase, a0, a1);
        uint32_t idx[CPT];
        bool ok[CPT];
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            const int ch = t + k * BT;
            ok[k] = has_row && ch < nch;
            idx[k] = rbase + min(ch, nch - 1) * 8;
        }
        // the residual first: its addresses need no pointer table, so its loads go out while the row's
        // table entries are still on their way (decode gather + norm 3.18 -> 3.04 us)
        uint4 rres[CPT];
        if (na.residual) {
#pragma unroll
            for (int k = 0; k < CPT; ++k) rres[k] = lds16(at(na.residual, 2 * idx[k]));
        }
        typename P::Raw raw[CPT];
#pragma unroll
        for (int k = 0; k < CPT; ++k) p.fetch(sh, pr, idx[k], raw[k], a0, a1);
        float h[CPT][8];
        float ss = 0.0f;
        float pk[CPT];
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            p.decode(raw[k], h[k], pr, idx[k], a0, a1);
            if (na.residual) {
                float rv[8];
                unpack_bf16x8(rres[k], rv);
#pragma unroll
                for (int e = 0; e < 8; ++e) h[k][e] = h[k][e] + rv[e];
            }
            if (na.residual_out && ok[k]) sts16(at(na.residual_out, 2 * idx[k]), pack_bf16x8(h[k]));
            if constexpr (kTreeSum) {
                float q = h[k][0] * h[k][0];
#pragma unroll
                for (int e = 1; e < 8; ++e) {
                    const float sq = h[k][e] * h[k][e];
                    q = q + sq;
                }
                pk[k] = ok[k] ? q : 0.0f;
            } else {
                float sk = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) sk = __builtin_fmaf(h[k][e], h[k][e], sk);
                ss += ok[k] ? sk : 0.0f;
            }
        }
        float tot = 0.0f;
        if constexpr (kTreeSum) {
#pragma unroll
            for (int k = 0; k < CPT; ++k) {
                const float ws = wave_sum(pk[k]);
                if (lane == 0) s_part[sub][k][wid] = ws;
            }
            __syncthreads();
            float lv[CPT];
#pragma unroll
            for (int k = 0; k < CPT; ++k) {
                float a[BT / 64];
#pragma unroll
                for (int w = 0; w < BT / 64; ++w) a[w] = s_part[sub][k][w];
#pragma unroll
                for (int width = BT / 64; width > 1; width /= 2)
#pragma unroll
                    for (int j = 0; j < width / 2; ++j) a[j] = a[2 * j] + a[2 * j + 1];
                lv[k] = a[0];
            }
#pragma unroll
            for (int width = CPT; width > 1; width /= 2)
#pragma unroll
                for (int j = 0; j < width / 2; ++j) lv[j] = lv[2 * j] + lv[2 * j + 1];
            tot = lv[0];
        } else {
            const float ws = wave_sum(ss);
            if (lane == 0) s_part[sub][0][wid] = ws;
            __syncthreads();
#pragma unroll
            for (int w = 0; w < BT / 64; ++w) tot += s_part[sub][0][w];
        }
        __syncthreads();
        const float ms = tot / (float)H;
        const float rinv = 1.0f / sqrtf(ms + na.eps);
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            float gk[8];
            uint4 gw = kHoistGamma ? g[k] : ld16(at(na.gamma, 2 * (idx[k] - rbase)));
            // Keeps the unpacking (and the wait for the gamma load) here: hoisted out of the row loop, it
            // would hold back every load of the first row until gamma has arrived.
            asm volatile("" : "+v"(gw.x), "+v"(gw.y), "+v"(gw.z), "+v"(gw.w));
            unpack_bf16x8(gw, gk);
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float a = h[k][e] * rinv;
                o[e] = a * gk[e];
            }
            if constexpr (P::kOutBits == 0) {
                if (ok[k]) sts16(at(na.out, 2 * idx[k]), pack_bf16x8(o));
            } else {
                p.store(pr, idx[k], o, ok[k], t + k * BT, a1);  // every lane: the group reduction needs them all
            }
        }
    }
}

// Threads per row and chunks per thread for a row of nch 8-element chunks.
struct RowShape {
    int bt, cpt;
};
// Lanes per row (bt) and 8-element chunks per lane (cpt).  With no more rows than compute units each
// row has a workgroup of its own and nothing else to overlap with, so the row is spread over as many
// lanes as possible (up to 1024, one chunk each); otherwise lanes take several chunks so that
// workgroups stay small enough to keep several resident per compute unit.
static RowShape row_shape(int64_t hidden, int64_t rows) {
    const int64_t nch = hidden / 8;
    if (rows <= 256 && nch > 256) {
        if (nch <= 512) return {512, 1};
        if (nch <= 1024) return {1024, 1};
        if (nch <= 2048) return {1024, 2};
    }
    if (nch <= 64) return {64, 1};
    if (nch <= 128) return {128, 1};
    if (nch <= 256) return {256, 1};
    if (nch <= 512) return {256, 2};
    if (nch <= 1024) return {256, 4};
    if (nch <= 2048) return {512, 4};
    if (nch <= 4096) return {1024, 4};
    return {1024, 8};
}

// grid: workgroups wanted (one per row, or the caller's cap).  A cap of at most a quarter of the rows
// on rows of at most 256 lanes puts several rows in flight per workgroup: 4, or 2 when each lane holds 4
// chunks (so that the loads in flight still fit in registers).
template <class P>
static hipError_t launch_rows(const P& p, uint32_t a0, int a1, const NormKArgs& na, int64_t rows, int grid,
                              hipStream_t s) {
    const RowShape rs = row_shape(na.hidden, rows);
    if (P::kOutBits == 0 && rs.bt <= 256 && (int64_t)grid * 4 <= rows) {
#define FC_ROWSN(BT, CPT, RPB)                                              \
        if (rs.bt == BT && rs.cpt == CPT) {                                 \
            k_rows<P, BT, CPT, RPB><<<grid, BT * RPB, 0, s>>>(rows, na.hidden, na.eps, na.gamma, na.residual, \
                                                               na.out, na.residual_out, a0, a1, p);       \
            return hipGetLastError();                                      \
        }
        if constexpr (P::kOutBits == 0) {  // capped grids: only the bf16-output producers take a cap
            FC_ROWSN(64, 1, 4)
            FC_ROWSN(128, 1, 4)
            FC_ROWSN(256, 1, 4)
            FC_ROWSN(256, 2, 4)
            FC_ROWSN(256, 4, 2)
        }
#undef FC_ROWSN
    }
#define FC_ROWS(BT, CPT)                                                    \
    if (rs.bt == BT && rs.cpt == CPT) {                                     \
        k_rows<P, BT, CPT, 1><<<grid, BT, 0, s>>>(rows, na.hidden, na.eps, na.gamma, na.residual, na.out, \
                                                  na.residual_out, a0, a1, p);                           \
        return hipGetLastError();                                          \
    }
    FC_ROWS(64, 1)
    FC_ROWS(128, 1)
    FC_ROWS(256, 1)
    FC_ROWS(256, 2)
    FC_ROWS(256, 4)
    FC_ROWS(512, 1)
    FC_ROWS(1024, 1)
    FC_ROWS(1024, 2)
    FC_ROWS(512, 4)
    FC_ROWS(1024, 4)
    FC_ROWS(1024, 8)
#undef FC_ROWS
    return hipErrorInvalidValue;
}

static NormKArgs norm_args(const NormParams& n) {
    return NormKArgs{n.residual, n.gamma, n.eps, (int)n.hidden, n.out, n.residual_out};
}

static int ilog2(int v) {
    int l = 0;
    while ((1 << l) < v) ++l;
    return l;
}

template <int BITS, bool UNIFORM>
static hipError_t gather_norm_layout(const GatherParams& p, const NormKArgs& na, int64_t rows, hipStream_t s) {
    GatherProducer<BITS, UNIFORM> g;
    for (int i = 0; i < kMaxRanks; ++i) {
        g.codes[i] = i < p.R ? p.codes[i] : nullptr;
        g.meta[i] = i < p.R ? p.meta[i] : nullptr;
    }
    return launch_rows(g, (uint32_t)p.L, ilog2(p.group), na, rows, (int)rows, s);
}

template <int BITS>
static hipError_t gather_norm_bits(const GatherParams& p, const NormKArgs& na, int64_t rows, hipStream_t s) {
    return (p.L % p.norm.hidden == 0) ? gather_norm_layout<BITS, true>(p, na, rows, s)
                                      : gather_norm_layout<BITS, false>(p, na, rows, s);
}

hipError_t launch_gather(const GatherParams& p, hipStream_t s) {
    if (p.y) {
        GatherKArgs a;
        for (int i = 0; i < kMaxRanks; ++i) {
            a.codes[i] = i < p.R ? p.codes[i] : nullptr;
            a.meta[i] = i < p.R ? p.meta[i] : nullptr;
        }
        a.L = p.L;
        a.nchunks = p.L / 8;
        a.log2g = ilog2(p.group);
        a.y = p.y;
        const dim3 grid((unsigned)((a.nchunks + 255) / 256), (unsigned)p.R);
        if (p.bits == 8) k_gather_plain<8><<<grid, 256, 0, s>>>(a);
        else k_gather_plain<4><<<grid, 256, 0, s>>>(a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (p.has_norm) {
        const int64_t rows = (int64_t)p.R * p.L / p.norm.hidden;
        return p.bits == 8 ? gather_norm_bits<8>(p, norm_args(p.norm), rows, s)
                           : gather_norm_bits<4>(p, norm_args(p.norm), rows, s);
    }
    return hipSuccess;
}

// =====================================================================================================
// Reduce-scatter receive side fused with the residual-add + RMSNorm, the normalized row quantized into
// the shard's all-gather message (the norm applied before the all-gather, TokenWeave, abstract).  One
// workgroup per row, one 16-element slot per lane (lane t owns elements [16t, 16t + 16) of the row):
// each rank's codes arrive in one 16-byte (8-bit) or 8-byte (4-bit) load and one scale/zero word, and
// the residual in two 16-byte loads.  The row's sum of squares takes the order fixed for quantized-output
// rows: 8-element chunk partials (left fold of h*h), then a pairwise tree over the chunk index c = 2t + j,
// i.e. the lane's two chunks, the lanes of the wavefront (DPP butterfly), then the wavefronts.  Rows of
// more than 1024 slots go through k_rows instead.
// =====================================================================================================
struct QNormTabs {
    // [shard in launch][rank]: entries past R repeat rank R-1
    const uint8_t* codes[kNormShards][kMaxRanks];
    const uint32_t* meta[kNormShards][kMaxRanks];
    uint8_t* out_codes[kNormShards];
    uint32_t* out_meta[kNormShards];
};
constexpr int kQNormMaxSlots = 1024;  // 16-element slots per row (H <= 16384)

// a1 = log2(group) | R << 8; L = shard length (a multiple of H); grid = rows, rows * H < 2^31.  One
// workgroup per row and no loop: loading the next row ahead into a second set of registers costs more
// occupancy than it hides, and a loop would let the compiler hoist gamma's unpacking (and the wait for
// it) in front of the first row's loads.
template <int B1, int B2, int BT, bool R8>
__global__ __launch_bounds__(BT) void k_reduce_norm(const int H, const float eps,
                                                    const uint16_t* __restrict__ gamma,
                                                    const uint16_t* residual, uint16_t* residual_out,
                                                    const uint32_t L, const int a1, const QNormTabs tb) {
    constexpr int E = 16;
    constexpr int IN_W = E * B1 / 32;  // code words per rank
    constexpr int RB = 8;              // ranks per batch of loads
    constexpr int NW = BT / 64;
    const int R = R8 ? 8 : (a1 >> 8);
    __builtin_assume(R >= 1);
    const int log2g = a1 & 0xff;
    const int nl = H / E;
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const bool ok = t < nl;
    const uint32_t e0 = (uint32_t)(ok ? t : nl - 1) * E;  // the slot's first element in the row
    __shared__ float s_part[NW];
    struct Where {
        uint32_t rbase, sh, off;  // row start, shard in the launch, element offset inside the shard
    };
    Where cw;
    cw.rbase = (uint32_t)blockIdx.x * (uint32_t)H;
    cw.sh = cw.rbase / L;
    cw.off = cw.rbase - cw.sh * L + e0;
    struct Batch {
        uint32_t wv[RB][IN_W];
        uint32_t mv[RB];
    };
    // byte offsets without a product that would pass 2^32 (off < 2^31)
    auto load_batch = [&](const Where& w, int r0, Batch& b) {
        const uint32_t coff = B1 == 8 ? w.off : w.off >> 1, moff = (w.off >> log2g) * 4u;
#pragma unroll
        for (int j = 0; j < RB; ++j) {
            load_codes<E, B1>(tb.codes[w.sh][r0 + j] + coff, b.wv[j]);
            b.mv[j] = lds4(reinterpret_cast<const uint8_t*>(tb.meta[w.sh][r0 + j]) + moff);
        }
    };
    auto load_residual = [&](const Where& w, uint4 (&rv)[2]) {
        if (residual) {
            rv[0] = lds16(residual + w.rbase + e0);
            rv[1] = lds16(residual + w.rbase + e0 + 8);
        }
    };
    float h[E];
    auto fold_batch = [&](const Batch& b, int r0) {
#pragma unroll
        for (int j = 0; j < RB; ++j) {
            if (r0 + j < R) {  // uniform
                float d[E];
#pragma unroll
                for (int w = 0; w < IN_W; ++w)
                    Unpack<B1>::run(b.wv[j][w], meta_scale(b.mv[j]), meta_zero(b.mv[j]), d + w * Unpack<B1>::PER_WORD);
                if (r0 + j == 0) {
#pragma unroll
                    for (int e = 0; e < E; ++e) h[e] = d[e];
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e) h[e] = h[e] + d[e];
                }
            }
        }
    };
    {
        Batch cb;
        uint4 cr[2] = {};
        uint8_t* const oc = tb.out_codes[cw.sh];  // read ahead of the loads, as in k_reduce (decode 4.66 -> 4.37 us)
        uint32_t* const om = tb.out_meta[cw.sh];
        load_batch(cw, 0, cb);
        load_residual(cw, cr);
        asm volatile("" ::"s"(oc), "s"(om));
        const uint4 g0 = ld16(gamma + e0), g1 = ld16(gamma + e0 + 8);  // gamma: shared by every row, an L2 hit
        fold_batch(cb, 0);
        for (int r0 = RB; r0 < R; r0 += RB) {  // more than 8 ranks
            Batch more;
            load_batch(cw, r0, more);
            fold_batch(more, r0);
        }
        if (residual) {
            float rv[8];
            unpack_bf16x8(cr[0], rv);
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = h[e] + rv[e];
            unpack_bf16x8(cr[1], rv);
#pragma unroll
            for (int e = 0; e < 8; ++e) h[8 + e] = h[8 + e] + rv[e];
        }
        if (residual_out && ok) {
            float a[8], b[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                a[e] = h[e];
                b[e] = h[8 + e];
            }
            // Write-back stores, not streamed: each of the two instructions fills every other 16 bytes of
            // the wavefront's span, and streamed halves left L2 before their other halves arrived (1.33x
            // the written bytes); in L2 the halves merge into whole lines.
            *reinterpret_cast<uint4*>(residual_out + cw.rbase + e0) = pack_bf16x8(a);
            *reinterpret_cast<uint4*>(residual_out + cw.rbase + e0 + 8) = pack_bf16x8(b);
        }
        float p[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            float q = h[8 * c] * h[8 * c];
#pragma unroll
            for (int e = 1; e < 8; ++e) {
                const float sq = h[8 * c + e] * h[8 * c + e];
                q = q + sq;
            }
            p[c] = q;
        }
        float tot = wave_sum(ok ? p[0] + p[1] : 0.0f);
        if constexpr (NW > 1) {
            if (lane == 0) s_part[wid] = tot;
            __syncthreads();
            float a[NW];
#pragma unroll
            for (int w = 0; w < NW; ++w) a[w] = s_part[w];
#pragma unroll
            for (int width = NW; width > 1; width /= 2)
#pragma unroll
                for (int j = 0; j < width / 2; ++j) a[j] = a[2 * j] + a[2 * j + 1];
            tot = a[0];
        }
        const float ms = tot / (float)H;
        const float rinv = 1.0f / sqrtf(ms + eps);
        float gk[E];
        {
            float gv[8];
            unpack_bf16x8(g0, gv);
#pragma unroll
            for (int e = 0; e < 8; ++e) gk[e] = gv[e];
            unpack_bf16x8(g1, gv);
#pragma unroll
            for (int e = 0; e < 8; ++e) gk[8 + e] = gv[e];
        }
        float o[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float a = h[e] * rinv;
            o[e] = a * gk[e];
        }
        auto quantize_store = [&](auto lpg) {
            constexpr int LPG = decltype(lpg)::value;
            uint32_t w[E * B2 / 32];
            uint32_t m;
            quantize_lane<B2, E, LPG>(o, w, m);  // every lane: the group reduction needs them all
            if (ok) {
                store_codes<E, B2>(oc + (B2 == 8 ? cw.off : cw.off >> 1), w);
                if ((t & (LPG - 1)) == 0) om[cw.off >> log2g] = m;
            }
        };
        switch (log2g) {  // uniform; a group spans G/16 lanes
            case 5: quantize_store(std::integral_constant<int, 2>{}); break;
            case 6: quantize_store(std::integral_constant<int, 4>{}); break;
            case 7: quantize_store(std::integral_constant<int, 8>{}); break;
            default: quantize_store(std::integral_constant<int, 16>{}); break;
        }
    }
}

template <int B1, int B2, bool R8>
static void reduce_norm_shape(int bt, int rows, const NormKArgs& na, uint32_t L, int a1, const QNormTabs& tb,
                              hipStream_t s) {
#define FC_QN(BT)                                                                                      \
    case BT:                                                                                           \
        if constexpr (BT < 1024 || R8)                                                                 \
            k_reduce_norm<B1, B2, BT, R8><<<rows, BT, 0, s>>>(na.hidden, na.eps, na.gamma, na.residual, \
                                                              na.residual_out, L, a1, tb);             \
        break;
    switch (bt) {
        FC_QN(64)
        FC_QN(128)
        FC_QN(256)
        FC_QN(512)
        FC_QN(1024)
    }
#undef FC_QN
}

template <int B1, int B2>
static hipError_t reduce_norm_bits(const ReduceNormQParams& q, hipStream_t s) {
    const ReduceParams& p = q.rs;
    const int64_t H = q.norm.hidden;
    // row indices are 32-bit: a launch covers at most kMaxElems-sized runs of whole shards
    const int64_t fit = (((int64_t)1 << 31) - 16) / (p.L > 0 ? p.L : 1);
    const int per = fit < kNormShards ? (fit > 0 ? (int)fit : 1) : kNormShards;
    for (int s0 = 0; s0 < p.n_shards; s0 += per) {
        const int ns = (p.n_shards - s0) < per ? (p.n_shards - s0) : per;
        QReduceProducer<B1, B2> prod;
        for (int i = 0; i < kNormShards; ++i) {
            const int si = s0 + (i < ns ? i : ns - 1);
            for (int r = 0; r < kMaxRanks; ++r) {
                const int t = si * p.R + (r < p.R ? r : p.R - 1);
                prod.codes[i][r] = p.in_codes[t];
                prod.meta[i][r] = p.in_meta[t];
            }
            prod.out_codes[i] = p.out_codes[si];
            prod.out_meta[i] = p.out_meta[si];
        }
        NormKArgs na = norm_args(q.norm);
        const int64_t off = (int64_t)s0 * p.L;
        if (na.residual) na.residual += off;
        if (na.residual_out) na.residual_out += off;
        na.out = nullptr;
        const int64_t rows = (int64_t)ns * p.L / H;
        const int a1 = ilog2(p.group) | (p.R << 8);
        hipError_t e;
        // one 16-element slot per lane; rows of more than 512 slots from other than 8 ranks take the
        // chunk-per-lane kernel (beside 1024 lanes, a second batch of rank loads does not fit in registers)
        if (H / 16 <= 512 || (H / 16 <= kQNormMaxSlots && p.R == 8)) {
            QNormTabs tb;
            for (int i = 0; i < kNormShards; ++i) {
                for (int r = 0; r < kMaxRanks; ++r) {
                    tb.codes[i][r] = prod.codes[i][r];
                    tb.meta[i][r] = prod.meta[i][r];
                }
                tb.out_codes[i] = prod.out_codes[i];
                tb.out_meta[i] = prod.out_meta[i];
            }
            int bt = 64;  // one 16-element slot per lane
            while (bt * 16 < H) bt *= 2;
            if (p.R == 8) reduce_norm_shape<B1, B2, true>(bt, (int)rows, na, (uint32_t)p.L, a1, tb, s);
            else reduce_norm_shape<B1, B2, false>(bt, (int)rows, na, (uint32_t)p.L, a1, tb, s);
            e = hipGetLastError();
        } else {
            e = launch_rows(prod, (uint32_t)p.L, a1, na, rows, (int)rows, s);
        }
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_reduce_norm(const ReduceNormQParams& q, hipStream_t s) {
    const int b1 = q.rs.bits_in, b2 = q.rs.bits_out;
    if (b1 == 8 && b2 == 8) return reduce_norm_bits<8, 8>(q, s);
    if (b1 == 4 && b2 == 8) return reduce_norm_bits<4, 8>(q, s);
    if (b1 == 8 && b2 == 4) return reduce_norm_bits<8, 4>(q, s);
    return reduce_norm_bits<4, 4>(q, s);
}

hipError_t launch_reduce_rmsnorm(const ReduceNormParams& p, hipStream_t s) {
    BF16ReduceProducer b;
    for (int i = 0; i < kMaxRanks; ++i) b.parts[i] = p.parts[i < p.R ? i : p.R - 1];
    const int64_t rows = p.rows;
    int grid = (int)rows;
    if (p.max_workgroups > 0 && p.max_workgroups < grid) grid = p.max_workgroups;
    return launch_rows(b, (uint32_t)p.R, 0, norm_args(p.norm), rows, grid, s);
}

}  // namespace fc
