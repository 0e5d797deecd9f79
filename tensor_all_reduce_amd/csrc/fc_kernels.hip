// fc_kernels.hip -- gfx950 kernels of the flash all-reduce path and their launchers.
//
// Every kernel streams HBM with 16-byte accesses per lane, keeps intermediate fp32 values in
// registers, and reduces across lanes with DPP (group min/max) or wave sums (RMSNorm).  None uses
// matrix cores: nothing on this path is a contraction.
#include "fc_device.h"
#include "fc_launch.h"

namespace fc {

// =====================================================================================================
// Group quantization (Flash Communication, summary "Core ideas of the solution": low-bit fine-grained
// quantization of activations).  One lane quantizes E consecutive elements: 16 for 8-bit codes, 32 for
// 4-bit codes, so that each lane writes exactly 16 bytes of codes; a group of G spans G/E lanes.
// =====================================================================================================
template <int BITS, int G>
__global__ __launch_bounds__(256) void k_quantize(const uint16_t* __restrict__ x, int64_t nchunks,
                                                  uint8_t* __restrict__ codes, uint32_t* __restrict__ meta) {
    constexpr int E = BITS == 8 ? 16 : 32;
    constexpr int LPG = G / E;
    const int64_t c0 = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const bool valid = c0 < nchunks;
    // Lanes past the end recompute the last chunk (whole groups lie on either side of the end), so every
    // lane of a DPP group holds valid data; only the stores are masked.
    const int64_t c = valid ? c0 : nchunks - 1;
    float v[E];
    const uint16_t* xp = x + c * E;
#pragma unroll
    for (int k = 0; k < E / 8; ++k) {
        const uint4 u = ld16(xp + 8 * k);
        v[8 * k + 0] = bf16_lo(u.x);
        v[8 * k + 1] = bf16_hi(u.x);
        v[8 * k + 2] = bf16_lo(u.y);
        v[8 * k + 3] = bf16_hi(u.y);
        v[8 * k + 4] = bf16_lo(u.z);
        v[8 * k + 5] = bf16_hi(u.z);
        v[8 * k + 6] = bf16_lo(u.w);
        v[8 * k + 7] = bf16_hi(u.w);
    }
    uint32_t w[E * BITS / 32];
    uint32_t m;
    quantize_lane<BITS, E, LPG>(v, w, m);
    if (valid) {
        st16(codes + c * 16, make_uint4(w[0], w[1], w[2], w[3]));
        if ((threadIdx.x % LPG) == 0) meta[c / LPG] = m;
    }
}

template <int BITS>
static hipError_t quantize_bits(const QuantizeParams& p, hipStream_t s) {
    constexpr int E = BITS == 8 ? 16 : 32;
    const int64_t nchunks = p.n / E;
    const dim3 grid((unsigned)((nchunks + 255) / 256));
    switch (p.group) {
        case 32: k_quantize<BITS, 32><<<grid, 256, 0, s>>>(p.x, nchunks, p.codes, p.meta); break;
        case 64: k_quantize<BITS, 64><<<grid, 256, 0, s>>>(p.x, nchunks, p.codes, p.meta); break;
        case 128: k_quantize<BITS, 128><<<grid, 256, 0, s>>>(p.x, nchunks, p.codes, p.meta); break;
        default: k_quantize<BITS, 256><<<grid, 256, 0, s>>>(p.x, nchunks, p.codes, p.meta); break;
    }
    return hipGetLastError();
}

hipError_t launch_quantize(const QuantizeParams& p, hipStream_t s) {
    return p.bits == 8 ? quantize_bits<8>(p, s) : quantize_bits<4>(p, s);
}

// =====================================================================================================
// Reduce-scatter receive side (two-step all-reduce, step one).  Block row y = shard; each lane owns E
// consecutive elements of the shard (E = 32 if either width is 4 bits, else 16), dequantizes them from
// every rank's message, folds them in fp32 in ascending rank order (flash-comm: reduction order fixed,
// independent of arrival order) and requantizes the fp32 sums for the all-gather step.
// =====================================================================================================
struct ReduceKArgs {
    const uint8_t* in_codes[kMaxReduceIn];
    const uint32_t* in_meta[kMaxReduceIn];
    uint8_t* out_codes[kMaxRanks];
    uint32_t* out_meta[kMaxRanks];
    int R;
    int64_t nchunks;  // lanes' chunks per shard = L / E
};

template <int B1, int B2, int G>
__global__ __launch_bounds__(256) void k_reduce(const ReduceKArgs a) {
    constexpr int E = (B1 == 4 || B2 == 4) ? 32 : 16;
    constexpr int LPG = G / E;
    constexpr int IN_BYTES = E * B1 / 8;   // 16 or 32
    constexpr int IN_W4 = IN_BYTES / 16;   // uint4 loads per rank
    constexpr int RB = 8;                  // ranks loaded per batch
    const int shard = blockIdx.y;
    const int64_t c0 = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const bool valid = c0 < a.nchunks;
    const int64_t c = valid ? c0 : a.nchunks - 1;
    const int64_t gidx = (c * E) / G;
    const int R = a.R;
    float acc[E];
    for (int r0 = 0; r0 < R; r0 += RB) {
        uint4 wv[RB][IN_W4];
        uint32_t mv[RB];
#pragma unroll
        for (int j = 0; j < RB; ++j) {
            if (r0 + j < R) {
                const int t = shard * R + r0 + j;
                const uint8_t* cp = a.in_codes[t] + c * IN_BYTES;
#pragma unroll
                for (int k = 0; k < IN_W4; ++k) wv[j][k] = ld16(cp + 16 * k);
                mv[j] = a.in_meta[t][gidx];
            }
        }
#pragma unroll
        for (int j = 0; j < RB; ++j) {
            if (r0 + j < R) {
                const float sc = meta_scale(mv[j]);
                const float z = meta_zero(mv[j]);
                float d[E];
                const uint32_t* ww = reinterpret_cast<const uint32_t*>(&wv[j][0]);
#pragma unroll
                for (int k = 0; k < E / Unpack<B1>::PER_WORD; ++k)
                    Unpack<B1>::run(ww[k], sc, z, d + k * Unpack<B1>::PER_WORD);
                if (r0 + j == 0) {
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[e] = d[e];
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[e] = acc[e] + d[e];
                }
            }
        }
    }
    constexpr int OW = E * B2 / 32;  // output words per lane: 4 or 8
    uint32_t w[OW];
    uint32_t m;
    quantize_lane<B2, E, LPG>(acc, w, m);
    if (valid) {
        uint8_t* op = a.out_codes[shard] + c * (OW * 4);
#pragma unroll
        for (int k = 0; k < OW / 4; ++k) st16(op + 16 * k, make_uint4(w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]));
        if ((threadIdx.x % LPG) == 0) a.out_meta[shard][c / LPG] = m;
    }
}

template <int B1, int B2>
static void reduce_launch_g(const ReduceKArgs& a, int group, dim3 grid, hipStream_t s) {
    switch (group) {
        case 32: k_reduce<B1, B2, 32><<<grid, 256, 0, s>>>(a); break;
        case 64: k_reduce<B1, B2, 64><<<grid, 256, 0, s>>>(a); break;
        case 128: k_reduce<B1, B2, 128><<<grid, 256, 0, s>>>(a); break;
        default: k_reduce<B1, B2, 256><<<grid, 256, 0, s>>>(a); break;
    }
}

hipError_t launch_reduce(const ReduceParams& p, hipStream_t s) {
    const int E = (p.bits_in == 4 || p.bits_out == 4) ? 32 : 16;
    const int64_t nchunks = p.L / E;
    const int per_launch = kMaxReduceIn / p.R;  // shards whose R pointers fit in one argument table
    for (int s0 = 0; s0 < p.n_shards; s0 += per_launch) {
        const int ns = (p.n_shards - s0) < per_launch ? (p.n_shards - s0) : per_launch;
        ReduceKArgs a;
        for (int i = 0; i < ns * p.R; ++i) {
            a.in_codes[i] = p.in_codes[s0 * p.R + i];
            a.in_meta[i] = p.in_meta[s0 * p.R + i];
        }
        for (int i = 0; i < ns; ++i) {
            a.out_codes[i] = p.out_codes[s0 + i];
            a.out_meta[i] = p.out_meta[s0 + i];
        }
        a.R = p.R;
        a.nchunks = nchunks;
        const dim3 grid((unsigned)((nchunks + 255) / 256), (unsigned)ns);
        if (p.bits_in == 8 && p.bits_out == 8) reduce_launch_g<8, 8>(a, p.group, grid, s);
        else if (p.bits_in == 4 && p.bits_out == 8) reduce_launch_g<4, 8>(a, p.group, grid, s);
        else if (p.bits_in == 8 && p.bits_out == 4) reduce_launch_g<8, 4>(a, p.group, grid, s);
        else reduce_launch_g<4, 4>(a, p.group, grid, s);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// =====================================================================================================
// All-gather receive side, plain mode: dequantize every shard to bf16.  Block row y = shard; each lane
// dequantizes the E codes held in 16 bytes (16 for 8-bit codes, 32 for 4-bit codes).
// =====================================================================================================
struct GatherKArgs {
    const uint8_t* codes[kMaxRanks];
    const uint32_t* meta[kMaxRanks];
    int64_t L;
    int64_t nchunks;  // per shard
    int log2g;
    uint16_t* y;
};

template <int BITS>
__global__ __launch_bounds__(256) void k_gather_plain(const GatherKArgs a) {
    constexpr int E = BITS == 8 ? 16 : 32;
    const int shard = blockIdx.y;
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= a.nchunks) return;
    const uint4 w = ld16(a.codes[shard] + c * 16);
    const uint32_t m = a.meta[shard][(c * E) >> a.log2g];
    const float sc = meta_scale(m), z = meta_zero(m);
    float d[E];
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) Unpack<BITS>::run(ww[k], sc, z, d + k * Unpack<BITS>::PER_WORD);
    uint16_t* yp = a.y + shard * a.L + c * E;
#pragma unroll
    for (int k = 0; k < E / 8; ++k)
        st16(yp + 8 * k, make_uint4(pack_bf16x2(d[8 * k], d[8 * k + 1]), pack_bf16x2(d[8 * k + 2], d[8 * k + 3]),
                                    pack_bf16x2(d[8 * k + 4], d[8 * k + 5]), pack_bf16x2(d[8 * k + 6], d[8 * k + 7])));
}

// =====================================================================================================
// Row kernels: produce the fp32 all-reduced value y of one row chunk by chunk (16 elements = 32 bytes of
// bf16 per lane and chunk), then apply the residual-add + RMSNorm epilogue (TokenWeave, abstract: fused
// AllReduce-RMSNorm).  A workgroup owns a row at a time, keeps h in registers (CPT chunks per lane),
// reduces sum(h^2) with DPP inside each wave and LDS across waves, and walks rows with a stride of the
// grid size so that the grid (the compute-unit footprint) can be capped.
// =====================================================================================================
struct NormKArgs {
    const uint16_t* residual;
    const uint16_t* gamma;
    float eps;
    int hidden;
    uint16_t* out;
    uint16_t* residual_out;
};

// y from the R requantized shards of the all-gather step.
template <int BITS>
struct GatherProducer {
    const uint8_t* codes[kMaxRanks];
    const uint32_t* meta[kMaxRanks];
    uint32_t L;
    int log2g;

    struct Shared {
        const uint8_t* codes[kMaxRanks];
        const uint32_t* meta[kMaxRanks];
    };
    __device__ void init(Shared& sh) const {
        if (threadIdx.x == 0) {
#pragma unroll
            for (int k = 0; k < kMaxRanks; ++k) {
                sh.codes[k] = codes[k];
                sh.meta[k] = meta[k];
            }
        }
    }
    __device__ __forceinline__ void load(const Shared& sh, uint32_t i, float (&y)[16]) const {
        const uint32_t s = i / L;  // a 16-element chunk never straddles a shard (L % 32 == 0)
        const uint32_t off = i - s * L;
        const uint32_t m = sh.meta[s][off >> log2g];
        const float sc = meta_scale(m), z = meta_zero(m);
        if constexpr (BITS == 8) {
            const uint4 w = ld16(sh.codes[s] + off);
            Unpack<8>::run(w.x, sc, z, y);
            Unpack<8>::run(w.y, sc, z, y + 4);
            Unpack<8>::run(w.z, sc, z, y + 8);
            Unpack<8>::run(w.w, sc, z, y + 12);
        } else {
            const uint2 w = ld8(sh.codes[s] + off / 2);
            Unpack<4>::run(w.x, sc, z, y);
            Unpack<4>::run(w.y, sc, z, y + 8);
        }
    }
};

// y from R bf16 partial sums, folded in fp32 in ascending rank order.
struct BF16ReduceProducer {
    const uint16_t* parts[kMaxRanks];
    int R;

    struct Shared {};
    __device__ void init(Shared&) const {}
    __device__ __forceinline__ void load(const Shared&, uint32_t i, float (&y)[16]) const {
        constexpr int RB = 8;
        for (int r0 = 0; r0 < R; r0 += RB) {
            uint4 a[RB], b[RB];
#pragma unroll
            for (int j = 0; j < RB; ++j) {
                if (r0 + j < R) {
                    a[j] = ld16(parts[r0 + j] + i);
                    b[j] = ld16(parts[r0 + j] + i + 8);
                }
            }
#pragma unroll
            for (int j = 0; j < RB; ++j) {
                if (r0 + j < R) {
                    const uint32_t w[8] = {a[j].x, a[j].y, a[j].z, a[j].w, b[j].x, b[j].y, b[j].z, b[j].w};
                    float v[16];
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        v[2 * k] = bf16_lo(w[k]);
                        v[2 * k + 1] = bf16_hi(w[k]);
                    }
                    if (r0 + j == 0) {
#pragma unroll
                        for (int e = 0; e < 16; ++e) y[e] = v[e];
                    } else {
#pragma unroll
                        for (int e = 0; e < 16; ++e) y[e] = y[e] + v[e];
                    }
                }
            }
        }
    }
};

__device__ __forceinline__ void unpack_bf16x16(uint4 a, uint4 b, float (&v)[16]) {
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        v[2 * k] = bf16_lo(w[k]);
        v[2 * k + 1] = bf16_hi(w[k]);
    }
}

__device__ __forceinline__ void store_bf16x16(uint16_t* p, const float (&v)[16]) {
    st16(p, make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                       pack_bf16x2(v[6], v[7])));
    st16(p + 8, make_uint4(pack_bf16x2(v[8], v[9]), pack_bf16x2(v[10], v[11]), pack_bf16x2(v[12], v[13]),
                           pack_bf16x2(v[14], v[15])));
}

template <class P, int BT, int CPT>
__global__ __launch_bounds__(BT) void k_rows(const P p, const NormKArgs na, int64_t rows) {
    __shared__ float s_part[BT / 64];
    __shared__ typename P::Shared sh;
    p.init(sh);
    __syncthreads();
    const int H = na.hidden;
    const int nch = H >> 4;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
        const uint32_t rbase = (uint32_t)(row * H);
        float h[CPT][16];
        float ss = 0.0f;
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            const int ch = threadIdx.x + k * BT;
            if (ch < nch) {
                const uint32_t i = rbase + ch * 16;
                p.load(sh, i, h[k]);
                if (na.residual) {
                    float rv[16];
                    unpack_bf16x16(ld16(na.residual + i), ld16(na.residual + i + 8), rv);
#pragma unroll
                    for (int e = 0; e < 16; ++e) h[k][e] = h[k][e] + rv[e];
                }
                if (na.residual_out) store_bf16x16(na.residual_out + i, h[k]);
#pragma unroll
                for (int e = 0; e < 16; ++e) ss = __builtin_fmaf(h[k][e], h[k][e], ss);
            }
        }
        const float ws = wave_sum(ss);
        if (lane == 0) s_part[wid] = ws;
        __syncthreads();
        float tot = 0.0f;
#pragma unroll
        for (int w = 0; w < BT / 64; ++w) tot += s_part[w];
        __syncthreads();
        const float ms = tot / (float)H;
        const float rinv = 1.0f / sqrtf(ms + na.eps);
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            const int ch = threadIdx.x + k * BT;
            if (ch < nch) {
                float g[16];
                unpack_bf16x16(ld16(na.gamma + ch * 16), ld16(na.gamma + ch * 16 + 8), g);
                float o[16];
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float a = h[k][e] * rinv;
                    o[e] = a * g[e];
                }
                store_bf16x16(na.out + rbase + ch * 16, o);
            }
        }
    }
}

// Threads per row and chunks per thread for a row of nch 16-element chunks.
struct RowShape {
    int bt, cpt;
};
static RowShape row_shape(int64_t hidden) {
    const int64_t nch = hidden / 16;
    if (nch <= 64) return {64, 1};
    if (nch <= 128) return {128, 1};
    if (nch <= 256) return {256, 1};
    if (nch <= 512) return {256, 2};
    if (nch <= 1024) return {256, 4};
    if (nch <= 2048) return {512, 4};
    return {1024, 4};
}

template <class P>
static hipError_t launch_rows(const P& p, const NormKArgs& na, int64_t rows, int grid, hipStream_t s) {
    const RowShape rs = row_shape(na.hidden);
#define FC_ROWS(BT, CPT)                                                    \
    if (rs.bt == BT && rs.cpt == CPT) {                                     \
        k_rows<P, BT, CPT><<<grid, BT, 0, s>>>(p, na, rows);                \
        return hipGetLastError();                                          \
    }
    FC_ROWS(64, 1)
    FC_ROWS(128, 1)
    FC_ROWS(256, 1)
    FC_ROWS(256, 2)
    FC_ROWS(256, 4)
    FC_ROWS(512, 4)
    FC_ROWS(1024, 4)
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

hipError_t launch_gather(const GatherParams& p, hipStream_t s) {
    if (p.y) {
        GatherKArgs a;
        for (int i = 0; i < kMaxRanks; ++i) {
            a.codes[i] = i < p.R ? p.codes[i] : nullptr;
            a.meta[i] = i < p.R ? p.meta[i] : nullptr;
        }
        const int E = p.bits == 8 ? 16 : 32;
        a.L = p.L;
        a.nchunks = p.L / E;
        a.log2g = ilog2(p.group);
        a.y = p.y;
        const dim3 grid((unsigned)((a.nchunks + 255) / 256), (unsigned)p.R);
        if (p.bits == 8) k_gather_plain<8><<<grid, 256, 0, s>>>(a);
        else k_gather_plain<4><<<grid, 256, 0, s>>>(a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (p.has_norm) {
        const NormKArgs na = norm_args(p.norm);
        const int64_t rows = (int64_t)p.R * p.L / p.norm.hidden;
        const int grid = (int)rows;
        if (p.bits == 8) {
            GatherProducer<8> g;
            for (int i = 0; i < kMaxRanks; ++i) {
                g.codes[i] = i < p.R ? p.codes[i] : nullptr;
                g.meta[i] = i < p.R ? p.meta[i] : nullptr;
            }
            g.L = (uint32_t)p.L;
            g.log2g = ilog2(p.group);
            return launch_rows(g, na, rows, grid, s);
        } else {
            GatherProducer<4> g;
            for (int i = 0; i < kMaxRanks; ++i) {
                g.codes[i] = i < p.R ? p.codes[i] : nullptr;
                g.meta[i] = i < p.R ? p.meta[i] : nullptr;
            }
            g.L = (uint32_t)p.L;
            g.log2g = ilog2(p.group);
            return launch_rows(g, na, rows, grid, s);
        }
    }
    return hipSuccess;
}

hipError_t launch_reduce_rmsnorm(const ReduceNormParams& p, hipStream_t s) {
    BF16ReduceProducer b;
    for (int i = 0; i < kMaxRanks; ++i) b.parts[i] = i < p.R ? p.parts[i] : nullptr;
    b.R = p.R;
    const int64_t rows = p.rows;
    int grid = (int)rows;
    if (p.max_workgroups > 0 && p.max_workgroups < grid) grid = p.max_workgroups;
    return launch_rows(b, norm_args(p.norm), rows, grid, s);
}

// =====================================================================================================
// Self-synchronizing slots (flash-comm, abstract): the receiver validates each block's epoch words
// itself, with no barrier.  Each lane owns 4 slots (32 bytes per rank, 8 output elements); a block of
// B slots spans LPB = B/4 aligned lanes, so its verdict is a field of a wavefront ballot.
// =====================================================================================================
struct LLKArgs {
    const uint64_t* slots[kMaxRanks];
    int R;
    int64_t nthreads;  // nslots / 4
    int64_t nblk;
    uint32_t epoch;
    uint16_t* out;
    uint8_t* stale;
    uint8_t* done;
    uint32_t* counters;
};

template <int LPB>
__global__ __launch_bounds__(256) void k_ll_unpack(const LLKArgs a) {
    __shared__ uint32_t s_cnt[2];
    if (threadIdx.x < 2) s_cnt[threadIdx.x] = 0;
    __syncthreads();
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int lane = threadIdx.x & 63;
    const bool valid = t < a.nthreads;
    const int64_t b = t / LPB;
    const bool leader = (lane % LPB) == 0;
    const bool active = valid && a.done[b] == 0;
    const uint64_t field = LPB == 64 ? ~0ull : ((1ull << LPB) - 1ull);
    const int shift = lane & ~(LPB - 1);
    float acc[8];
    bool all_valid = true;
    uint32_t n_stale = 0;
    for (int r = 0; r < a.R; ++r) {
        uint4 s0 = make_uint4(0, a.epoch, 0, a.epoch), s1 = s0;
        if (active) {
            const uint64_t* sp = a.slots[r] + 4 * t;
            s0 = ld16(sp);
            s1 = ld16(sp + 2);
        }
        // slot = {payload dword, epoch dword}: epoch words are .y and .w of each 16-byte load
        const bool st = (s0.y != a.epoch) | (s0.w != a.epoch) | (s1.y != a.epoch) | (s1.w != a.epoch);
        const uint64_t bal = __ballot(st);
        const bool blk_stale = ((bal >> shift) & field) != 0;
        if (active && leader) {
            a.stale[(int64_t)r * a.nblk + b] = blk_stale ? 1 : 0;
            n_stale += blk_stale ? 1u : 0u;
        }
        all_valid = all_valid && !blk_stale;
        const float v[8] = {bf16_lo(s0.x), bf16_hi(s0.x), bf16_lo(s0.z), bf16_hi(s0.z),
                            bf16_lo(s1.x), bf16_hi(s1.x), bf16_lo(s1.z), bf16_hi(s1.z)};
        if (r == 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = v[e];
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = acc[e] + v[e];
        }
    }
    uint32_t n_pending = 0;
    if (active) {
        if (all_valid) {
            st16(a.out + 8 * t, make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                           pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])));
            if (leader) a.done[b] = 1;
        } else if (leader) {
            n_pending = 1;
        }
    }
    if (n_stale) atomicAdd(&s_cnt[0], n_stale);
    if (n_pending) atomicAdd(&s_cnt[1], n_pending);
    __syncthreads();
    if (threadIdx.x < 2 && s_cnt[threadIdx.x]) atomicAdd(&a.counters[threadIdx.x], s_cnt[threadIdx.x]);
}

hipError_t launch_ll_unpack(const LLParams& p, hipStream_t s) {
    LLKArgs a;
    for (int i = 0; i < kMaxRanks; ++i) a.slots[i] = i < p.R ? p.slots[i] : nullptr;
    a.R = p.R;
    const int64_t nslots = p.n / 2;
    a.nthreads = nslots / 4;
    a.nblk = nslots / p.block_slots;
    a.epoch = p.epoch;
    a.out = p.out;
    a.stale = p.stale;
    a.done = p.done;
    a.counters = p.counters;
    const dim3 grid((unsigned)((a.nthreads + 255) / 256));
    switch (p.block_slots) {
        case 32: k_ll_unpack<8><<<grid, 256, 0, s>>>(a); break;
        case 64: k_ll_unpack<16><<<grid, 256, 0, s>>>(a); break;
        case 128: k_ll_unpack<32><<<grid, 256, 0, s>>>(a); break;
        default: k_ll_unpack<64><<<grid, 256, 0, s>>>(a); break;
    }
    return hipGetLastError();
}

// Sender emulation: lane j of the write order packs 4 slots of block order[j / LPB].
// An order entry outside [0, nblk) (not a permutation: out of contract) writes nothing.
__global__ __launch_bounds__(256) void k_ll_pack(const uint16_t* __restrict__ x, int64_t nthreads, int lpb,
                                                 int block_slots, const int32_t* __restrict__ order, uint32_t epoch,
                                                 uint64_t* __restrict__ slots) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= nthreads) return;
    const int64_t j = t / lpb;
    const int64_t b = order ? (int64_t)order[j] : j;
    if (b < 0 || b >= nthreads / lpb) return;
    const int64_t k0 = b * block_slots + 4 * (t % lpb);
    const uint4 xv = ld16(x + 2 * k0);
    st16(slots + k0, make_uint4(xv.x, epoch, xv.y, epoch));
    st16(slots + k0 + 2, make_uint4(xv.z, epoch, xv.w, epoch));
}

hipError_t launch_ll_pack(const PackParams& p, hipStream_t s) {
    const int64_t nthreads = p.n / 8;
    const dim3 grid((unsigned)((nthreads + 255) / 256));
    k_ll_pack<<<grid, 256, 0, s>>>(p.x, nthreads, p.block_slots / 4, p.block_slots, p.order, p.epoch, p.slots);
    return hipGetLastError();
}

// =====================================================================================================
// Copy ceiling: 16-byte loads and stores, 4 per lane per iteration, grid-stride.
// =====================================================================================================
__global__ __launch_bounds__(256) void k_copy(const uint4* __restrict__ src, uint4* __restrict__ dst, int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * 256 * 4;
    for (int64_t base = (int64_t)blockIdx.x * 256 * 4 + threadIdx.x; base < n16; base += stride) {
        uint4 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (base + k * 256 < n16) v[k] = src[base + k * 256];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (base + k * 256 < n16) dst[base + k * 256] = v[k];
    }
}

hipError_t launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t s) {
    const int64_t n16 = bytes / 16;
    int64_t blocks = (n16 + 1023) / 1024;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) blocks = 1;
    k_copy<<<(unsigned)blocks, 256, 0, s>>>(reinterpret_cast<const uint4*>(src), reinterpret_cast<uint4*>(dst), n16);
    return hipGetLastError();
}

}  // namespace fc
