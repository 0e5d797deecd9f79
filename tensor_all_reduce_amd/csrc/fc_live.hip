// fc_live.hip -- gfx950 kernels of the readiness encodings that a receiver reads while the senders are
// still writing (flash-comm, abstract: each block carries evidence of its readiness, and the protocol
// selector picks how that evidence is encoded):
//   * one flag word per block: the sender stores the block's payload, then the epoch into the block's
//     flag with release order; the receiver reads the flag, fences with acquire order, then the payload;
//   * 8-byte slots (payload word + epoch word) read by a polling receiver with atomic 64-bit loads.
// Every wait is bounded by a poll budget, so every kernel ends whether or not its sender finishes; what
// is still stale at the last look is left pending for a later call.
#include "fc_device.h"
#include "fc_launch.h"
#include "fc_sync.h"

namespace fc {

// =====================================================================================================
// Flag encoding, sender side: R peers writing at the same time, grid row y = rank.  A workgroup writes a
// span of K consecutive entries of the write order (K blocks: the span is chosen by the launcher from the
// message size, 2^13 to 2^17 elements, and K = 1 for blocks as large as the span), 16 bytes per lane, then
// publishes them: a barrier (which orders every wave's stores before it at workgroup scope), one release
// fence at agent scope by the first wavefront, which writes the span back past its XCD's L2, and the K
// flag stores.  The fence is the expensive step (it writes back the L2), so one fence covers a whole span
// rather than each block.
// =====================================================================================================
struct FlagPackTabs {
    const uint16_t* x[kMaxRanks];
    const int32_t* order[kMaxRanks];
    uint16_t* payload[kMaxRanks];
    uint32_t* flags[kMaxRanks];
};

__global__ __launch_bounds__(256) void k_flag_pack(const int64_t nblk, const int log2_be, const int log2_k,
                                                   const uint32_t epoch, const int pace, const FlagPackTabs t) {
    const int r = blockIdx.y;
    const uint16_t* x = t.x[r];
    const int32_t* order = t.order[r];
    uint16_t* payload = t.payload[r];
    uint32_t* flags = t.flags[r];
    const int64_t be = int64_t(1) << log2_be;
    const int64_t nspan = (nblk + (1 << log2_k) - 1) >> log2_k;
    for (int64_t j = blockIdx.x; j < nspan; j += gridDim.x) {  // trip count uniform over the workgroup
        pace_sleep(pace);
        for (int64_t e = (int64_t)threadIdx.x * 8; e < (be << log2_k); e += 256 * 8) {
            const int64_t q = (j << log2_k) + (e >> log2_be);  // entry of the write order
            if (q >= nblk) break;                                // ragged last span
            const int64_t b = order ? (int64_t)order[q] : q;
            if (b < 0 || b >= nblk) continue;  // not a permutation: out of contract, nothing written
            const int64_t i = (b << log2_be) + (e & (be - 1));
            *reinterpret_cast<uint4*>(payload + i) = ld16(x + i);
        }
        // The barrier orders every wave's stores before the first wavefront's fence at workgroup scope,
        // and the fence at agent scope is cumulative; each wave also waits here until its own stores have
        // reached the L2, so the write-back that the fence starts sees the whole span.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (threadIdx.x < 64) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            for (int k = threadIdx.x; k < (1 << log2_k); k += 64) {  // the span's K flags, 64 at a time
                const int64_t q = (j << log2_k) + k;
                if (q >= nblk) break;
                const int64_t b = order ? (int64_t)order[q] : q;
                if (b >= 0 && b < nblk) __hip_atomic_store(flags + b, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

hipError_t launch_flag_pack(const FlagPackParams& p, hipStream_t s) {
    FlagPackTabs t;
    for (int i = 0; i < kMaxRanks; ++i) {
        const int q = i < p.R ? i : p.R - 1;
        t.x[i] = p.x[q];
        t.order[i] = p.order[q];
        t.payload[i] = p.payload[q];
        t.flags[i] = p.flags[q];
    }
    const int64_t nblk = p.n >> p.log2_block;
    // Span of one fence: about a 32nd of the message, between 2^13 and 2^17 elements (never less than a
    // block).  Larger spans mean fewer L2 writebacks; smaller ones more workgroups and earlier flags.
    int log2_span = 13;
    while (log2_span < 17 && (int64_t(1) << (log2_span + 5)) < p.n) ++log2_span;
    const int log2_k = p.log2_block >= log2_span ? 0 : log2_span - p.log2_block;
    const int64_t nspan = (nblk + (1 << log2_k) - 1) >> log2_k;
    const dim3 grid((unsigned)(nspan < 2048 ? nspan : 2048), (unsigned)p.R);
    k_flag_pack<<<grid, 256, 0, s>>>(nblk, p.log2_block, log2_k, p.epoch, p.pace, t);
    return hipGetLastError();
}

// =====================================================================================================
// Flag encoding, receiver side.  A workgroup owns tiles of max(block, 2048) elements (NBW = 4, 2 or 1
// whole blocks), walked with a grid stride.  Its first wavefront checks the readiness evidence: lane
// (q, r) = (lane / 16, lane % 16) reads rank r's flag of the tile's block q with an agent-scope atomic
// load, re-reads the flags after a short sleep while a copy is stale and the budget lasts, fences once
// with acquire order and posts the verdicts in LDS.  After a barrier (which carries the acquire to the
// other wavefronts), all four wavefronts read the valid blocks' payload, 512 elements per instruction
// (16 bytes per lane, 8 ranks' loads in flight, the launcher repeating the last rank's pointer past R),
// and fold it in ascending rank order.  A stale copy's payload is never read.  One fence per tile and
// the whole workgroup on one block keep both the fences and the dependent flag-then-payload round trip
// per byte low.
// =====================================================================================================
struct FlagTabs {
    const uint16_t* payload[kMaxRanks];
    const uint32_t* flags[kMaxRanks];
};

template <int NBW>
__global__ __launch_bounds__(256) void k_flag_unpack(const int64_t ntiles, const int64_t nblk, const int log2_be,
                                                     const uint32_t epoch, const int R, const int max_polls,
                                                     uint8_t* done, uint16_t* out, uint8_t* stale,
                                                     uint32_t* counters, const FlagTabs t) {
    constexpr int RB = 8;  // ranks per batch of payload loads
    __shared__ uint64_t s_bad[2], s_watch[2];  // verdicts, double-buffered by tile parity
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int q = lane >> 4, rk = lane & 15;
    const uint32_t* fp = t.flags[rk < R ? rk : R - 1];
    const int log2_te = NBW > 1 ? 11 : log2_be;  // tile elements
    const int per_wave = 1 << (log2_te - 11);     // 512-element instructions per wavefront and tile
    uint32_t n_stale = 0, n_pending = 0, n_polls = 0;
    int par = 0;
    // The first wavefront reads a tile's flag words and done bytes one tile ahead: the next tile's are
    // issued before this tile's payload loads, so their round trip overlaps this tile's payload.
    auto flag_word = [&](int64_t b0) {
        const int64_t qb = b0 + (q < NBW ? q : NBW - 1);
        return qb < nblk ? qb : nblk - 1;  // this lane's flag word (clamped, always inside)
    };
    uint32_t f_next = 0;
    uint8_t d_next = 1;
    if (wave == 0 && (int64_t)blockIdx.x < ntiles) {
        const int64_t fb = flag_word((int64_t)blockIdx.x * NBW);
        f_next = ld_relaxed(fp + fb);
        d_next = done[fb];
    }
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x, par ^= 1) {  // uniform over the workgroup
        const int64_t b0 = tile * NBW;
        if (wave == 0) {
            const int64_t fb = flag_word(b0);
            const bool watch = q < NBW && rk < R && b0 + q < nblk && d_next == 0;
            uint32_t f = f_next;
            uint64_t bad = __ballot(watch && f != epoch);
            for (int p = 0; bad != 0 && p < max_polls; ++p) {
                __builtin_amdgcn_s_sleep(2);
                f = ld_relaxed(fp + fb);
                bad = __ballot(watch && f != epoch);
                ++n_polls;
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            if (watch) stale[(int64_t)rk * nblk + fb] = f != epoch ? 1 : 0;
            const uint64_t wm = __ballot(watch);
            if (lane == 0) {
                s_bad[par] = bad;
                s_watch[par] = wm;
            }
            n_stale += (uint32_t)__builtin_popcountll(bad);
#pragma unroll
            for (int k = 0; k < NBW; ++k)
                n_pending += ((wm >> (16 * k)) & 1u) && ((bad >> (16 * k)) & 0xffffu) ? 1u : 0u;
            // block `lane` of the tile is done when examined (its rank-0 lane watched) with no stale copy
            if (lane < NBW && ((wm >> (16 * lane)) & 1u) && ((bad >> (16 * lane)) & 0xffffu) == 0) done[b0 + lane] = 1;
            const int64_t nt = tile + (int64_t)gridDim.x;
            if (nt < ntiles) {  // uniform
                const int64_t nfb = flag_word(nt * NBW);
                f_next = ld_relaxed(fp + nfb);
                d_next = done[nfb];
            }
        }
        __syncthreads();
        const uint64_t bad = s_bad[par], wm = s_watch[par];
        bool valid[NBW];  // wavefront-uniform
#pragma unroll
        for (int k = 0; k < NBW; ++k) valid[k] = ((wm >> (16 * k)) & 1u) && ((bad >> (16 * k)) & 0xffffu) == 0;
        bool any = false;
#pragma unroll
        for (int k = 0; k < NBW; ++k) any = any || valid[k];
        if (!any) continue;
        const int64_t tbase = tile << log2_te;
        for (int j = 0; j < per_wave; j += 2) {
            // this wavefront's instructions i = wave + 4 j (+ 4): block (i * 512) >> log2_be of the tile
            bool vk[2];
            int64_t e0[2];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int i = wave + 4 * (j + k);
                const int kb = (i << 9) >> log2_be;
                bool v = false;
#pragma unroll
                for (int c = 0; c < NBW; ++c) v = v || (kb == c && valid[c]);
                vk[k] = j + k < per_wave && v;
                e0[k] = tbase + (int64_t)i * 512 + lane * 8;
            }
            float acc[2][8];
            auto batch = [&](int r0, bool first) {
                uint4 sv[RB][2];
#pragma unroll
                for (int jr = 0; jr < RB; ++jr)
#pragma unroll
                    for (int k = 0; k < 2; ++k)
                        if (vk[k]) sv[jr][k] = lds16(t.payload[r0 + jr] + e0[k]);
#pragma unroll
                for (int jr = 0; jr < RB; ++jr) {
                    if (r0 + jr >= R) continue;
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        if (!vk[k]) continue;
                        const uint32_t w[4] = {sv[jr][k].x, sv[jr][k].y, sv[jr][k].z, sv[jr][k].w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float lo = bf16_lo(w[e]), hi = bf16_hi(w[e]);
                            acc[k][2 * e] = first && jr == 0 ? lo : acc[k][2 * e] + lo;
                            acc[k][2 * e + 1] = first && jr == 0 ? hi : acc[k][2 * e + 1] + hi;
                        }
                    }
                }
            };
            batch(0, true);
            for (int r0 = RB; r0 < R; r0 += RB) batch(r0, false);
#pragma unroll
            for (int k = 0; k < 2; ++k)
                if (vk[k])
                    sts16(out + e0[k],
                          make_uint4(pack_bf16x2(acc[k][0], acc[k][1]), pack_bf16x2(acc[k][2], acc[k][3]),
                                     pack_bf16x2(acc[k][4], acc[k][5]), pack_bf16x2(acc[k][6], acc[k][7])));
        }
    }
    // wave 0 holds the counts: stale pairs and pending blocks in one 64-bit atomic (a call adds at most 2^29
    // stale pairs, so the low word does not carry), re-reads in one 32-bit atomic
    if (threadIdx.x == 0 && counters != nullptr) {  // counters == NULL: nothing is counted
        uint32_t* const cg = counter_group(counters);
        if (n_stale | n_pending)
            atomicAdd(reinterpret_cast<unsigned long long*>(cg), ((unsigned long long)n_pending << 32) | n_stale);
        if (n_polls) atomicAdd(cg + 2, n_polls);
    }
}

namespace {
unsigned poll_grid(int64_t ntiles, int max_workgroups) {
    const int64_t wgs = (ntiles + 3) / 4;  // 4 wavefronts per workgroup, one tile each
    return (unsigned)(max_workgroups > 0 && wgs > max_workgroups ? max_workgroups : wgs);
}
}  // namespace

hipError_t launch_flag_unpack(const FlagParams& p, hipStream_t s) {
    FlagTabs t;
    for (int i = 0; i < kMaxRanks; ++i) {
        t.payload[i] = p.payload[i < p.R ? i : p.R - 1];
        t.flags[i] = p.flags[i < p.R ? i : p.R - 1];
    }
    const int64_t nblk = p.n >> p.log2_block;
    const int nbw = p.log2_block >= 11 ? 1 : 1 << (11 - p.log2_block);  // blocks per workgroup tile
    const int64_t ntiles = (nblk + nbw - 1) / nbw;
    const unsigned grid =
        (unsigned)(p.poll.max_workgroups > 0 && ntiles > p.poll.max_workgroups ? p.poll.max_workgroups : ntiles);
#define FC_FU(NBW)                                                                                             \
    k_flag_unpack<NBW><<<grid, 256, 0, s>>>(ntiles, nblk, p.log2_block, p.epoch, p.R, p.poll.max_polls, p.done, \
                                            p.out, p.stale, p.counters, t)
    switch (nbw) {
        case 4: FC_FU(4); break;
        case 2: FC_FU(2); break;
        default: FC_FU(1); break;
    }
#undef FC_FU
    return hipGetLastError();
}

// =====================================================================================================
// Polling receiver of the 8-byte slots.  A wavefront owns tiles of 256 slots (4 instructions of 64
// slots, 8 bytes per lane), walked with a grid stride; every slot is read with an agent-scope atomic
// 64-bit load, so payload and epoch word are seen together and no fence is needed.  While a rank has a
// stale block in the tile and the budget lasts, that rank's slots of the tile are read again after a
// short sleep.  Verdicts (bit r of vs[b] = rank r's copy of tile block b is stale), fold and outputs as
// for the one-look receiver; all verdicts are wavefront-uniform.
// =====================================================================================================
template <int B>
__global__ __launch_bounds__(256) void k_ll_poll(const int64_t nslots, const int64_t nblk, const int64_t ntiles,
                                                 const uint32_t epoch, const int R, const int max_polls,
                                                 uint8_t* done, uint16_t* out, uint8_t* stale, uint32_t* counters,
                                                 const LLSlots t) {
    constexpr int NBT = 256 / B;  // blocks per tile: 8, 4, 2 or 1
    __shared__ uint32_t s_cnt[4][3];
    const int lane = threadIdx.x & 63;
    uint32_t n_stale = 0, n_pending = 0, n_polls = 0;
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    for (int64_t tile = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); tile < ntiles; tile += nwaves) {
        const int64_t s0 = tile * 256, b0 = tile * NBT;
        // blocks of the tile to examine (bit b = block b0 + b): inside the buffer and not done yet
        const int64_t qa = b0 + (lane < NBT ? lane : 0);
        const int64_t qb = qa < nblk ? qa : nblk - 1;
        const uint32_t act = (uint32_t)__ballot(lane < NBT && b0 + lane < nblk && done[qb] == 0);
        if (act == 0) continue;
        // byte offset of this lane's slot of instruction k from the tile's first slot (clamped inside the
        // buffer): a wavefront-uniform base plus a 32-bit lane offset, the same for every rank
        uint32_t off[4];
        bool on[4];  // this lane's slot of instruction k lies in a block to examine
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t sl = s0 + k * 64 + lane;
            off[k] = (uint32_t)((sl < nslots ? sl : nslots - 1) - s0) * 8u;
            on[k] = sl < nslots && ((act >> ((k * 64 + lane) / B)) & 1u);
        }
        // w[r][k]: payload word of rank r's slot; the epoch words are examined as soon as they arrive
        uint32_t w[kMaxRanks][4];
        uint32_t vs[NBT] = {};
        uint32_t need = (1u << R) - 1u;  // ranks whose slots are (re)read
        for (int p = 0;; ++p) {
            // opaque to the optimizer, so that the 16 x 4 slot addresses are not hoisted out of the loop
            // and kept in registers
            asm volatile("" : "+v"(off[0]), "+v"(off[1]), "+v"(off[2]), "+v"(off[3]));
#pragma unroll
            for (int r = 0; r < kMaxRanks; ++r) {
                if (!((need >> r) & 1u)) continue;  // uniform
                const char* base = reinterpret_cast<const char*>(t.p[r] + s0);
                uint32_t ep[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint64_t v = ld_relaxed(reinterpret_cast<const uint64_t*>(base + off[k]));
                    w[r][k] = (uint32_t)v;
                    ep[k] = (uint32_t)(v >> 32);
                }
#pragma unroll
                for (int b = 0; b < NBT; ++b) vs[b] &= ~(1u << r);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint64_t bal = __ballot(on[k] && ep[k] != epoch);
                    uint32_t lo = (uint32_t)bal, hi = (uint32_t)(bal >> 32);
                    asm("" : "+s"(lo), "+s"(hi));
                    if constexpr (B == 32) {
                        vs[2 * k] |= s_nonzero(lo) << r;
                        vs[2 * k + 1] |= s_nonzero(hi) << r;
                    } else {
                        vs[k * 64 / B] |= s_nonzero(lo | hi) << r;
                    }
                }
            }
            need = 0;
#pragma unroll
            for (int b = 0; b < NBT; ++b) need |= vs[b];
            if (need == 0 || p >= max_polls) break;
            ++n_polls;
            __builtin_amdgcn_s_sleep(2);
        }
        // fold in ascending rank order, store the lanes of valid blocks
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float a0 = 0.f, a1 = 0.f;
#pragma unroll
            for (int r = 0; r < kMaxRanks; ++r) {
                if (r >= R) continue;
                a0 = r == 0 ? bf16_lo(w[r][k]) : a0 + bf16_lo(w[r][k]);
                a1 = r == 0 ? bf16_hi(w[r][k]) : a1 + bf16_hi(w[r][k]);
            }
            uint32_t sm;  // this lane's block verdict, selected with masks
            if constexpr (B == 32) {
                const uint32_t h = 0u - (uint32_t)(lane >> 5);
                sm = (vs[2 * k] & ~h) | (vs[2 * k + 1] & h);
            } else {
                sm = vs[k * 64 / B];
            }
            if (on[k] && sm == 0) sts4(out + 2 * (s0 + k * 64 + lane), pack_bf16x2(a0, a1));
        }
        // per block: stale flags (lane r writes rank r's), done, counters
#pragma unroll
        for (int b = 0; b < NBT; ++b) {
            if (!((act >> b) & 1u)) continue;
            if (lane < R) stale[(int64_t)lane * nblk + b0 + b] = (vs[b] >> lane) & 1u;
            if (lane == 0 && vs[b] == 0) done[b0 + b] = 1;
            n_pending += s_nonzero(vs[b]);
            n_stale += (uint32_t)__builtin_popcount(vs[b]);
        }
    }
    if (counters == nullptr) return;  // uniform: nothing is counted
    if (lane == 0) {
        s_cnt[threadIdx.x >> 6][0] = n_stale;
        s_cnt[threadIdx.x >> 6][1] = n_pending;
        s_cnt[threadIdx.x >> 6][2] = n_polls;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t st = s_cnt[0][0] + s_cnt[1][0] + s_cnt[2][0] + s_cnt[3][0];
        const uint32_t pe = s_cnt[0][1] + s_cnt[1][1] + s_cnt[2][1] + s_cnt[3][1];
        const uint32_t po = s_cnt[0][2] + s_cnt[1][2] + s_cnt[2][2] + s_cnt[3][2];
        uint32_t* const cg = counter_group(counters);
        if (st | pe) atomicAdd(reinterpret_cast<unsigned long long*>(cg), ((unsigned long long)pe << 32) | st);
        if (po) atomicAdd(cg + 2, po);
    }
}

hipError_t launch_ll_poll(const LLParams& p, const PollParams& q, hipStream_t s) {
    LLSlots t;
    for (int i = 0; i < kMaxRanks; ++i) t.p[i] = p.slots[i < p.R ? i : p.R - 1];
    const int64_t nslots = p.n / 2, nblk = nslots / p.block_slots, ntiles = (nslots + 255) / 256;
    const unsigned grid = poll_grid(ntiles, q.max_workgroups);
#define FC_LLP(B) \
    k_ll_poll<B><<<grid, 256, 0, s>>>(nslots, nblk, ntiles, p.epoch, p.R, q.max_polls, p.done, p.out, p.stale, p.counters, t)
    switch (p.block_slots) {
        case 32: FC_LLP(32); break;
        case 64: FC_LLP(64); break;
        case 128: FC_LLP(128); break;
        default: FC_LLP(256); break;
    }
#undef FC_LLP
    return hipGetLastError();
}

}  // namespace fc
