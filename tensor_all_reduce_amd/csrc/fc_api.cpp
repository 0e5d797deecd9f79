// fc_api.cpp -- the C ABI declared in include/fc.h: argument validation on the host, then kernel launch.
// No call allocates, frees or synchronizes; every check runs before the first HIP call, so invalid
// arguments are reported without touching the device.
#include "fc.h"

#include <stdint.h>

#include "fc_launch.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxElems = (int64_t(1) << 31) - 16;  // per rank buffer; kernels index in 32 bits
constexpr int64_t kMaxHidden = 65536;

bool valid_bits(int b) { return b == 4 || b == 8; }
bool valid_group(int g) { return g == 32 || g == 64 || g == 128 || g == 256; }
bool valid_block(int b) { return b == 32 || b == 64 || b == 128 || b == 256; }
constexpr int kMaxPolls = 1 << 20;  // re-reads per tile of a polling receiver
constexpr int kMaxPace = 1 << 16;   // sender sleeps per block

// log2 of a flag-encoding block (a power of two from 512 to 65536 elements), or -1
int log2_flag_block(int b) {
    for (int l = 9; l <= 16; ++l)
        if (b == (1 << l)) return l;
    return -1;
}
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};
Range rng(const void* p, int64_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + (uintptr_t)bytes};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

fc_status launched(hipError_t e) {
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return FC_E_LAUNCH;
    }
    return FC_OK;
}

// Validation shared by the two epilogue users.  rows*hidden = n elements.
fc_status check_norm(const fc_norm* nm, int64_t n) {
    if (!nm->gamma || !nm->out) return FC_E_NULL;
    if (!(nm->eps > 0.0f) || nm->eps != nm->eps || nm->eps > 3.0e38f) return FC_E_ARG;
    if (nm->hidden <= 0 || nm->hidden % 8 != 0 || nm->hidden > kMaxHidden || n % nm->hidden != 0) return FC_E_SHAPE;
    if (!aligned(nm->gamma, 16) || !aligned(nm->out, 16) || (nm->residual && !aligned(nm->residual, 16)) ||
        (nm->residual_out && !aligned(nm->residual_out, 16)))
        return FC_E_ALIGN;
    const Range out = rng(nm->out, 2 * n);
    const Range g = rng(nm->gamma, 2 * nm->hidden);
    if (overlap(out, g)) return FC_E_ARG;
    if (nm->residual && overlap(out, rng(nm->residual, 2 * n))) return FC_E_ARG;
    if (nm->residual_out) {
        const Range ro = rng(nm->residual_out, 2 * n);
        if (overlap(ro, out) || overlap(ro, g)) return FC_E_ARG;
        if (nm->residual && nm->residual != nm->residual_out && overlap(ro, rng(nm->residual, 2 * n))) return FC_E_ARG;
    }
    return FC_OK;
}

fc::NormParams norm_params(const fc_norm* nm) {
    return fc::NormParams{nm->residual, nm->gamma, nm->eps, nm->hidden, nm->out, nm->residual_out};
}

}  // namespace

extern "C" {

int fc_abi_version(void) { return FC_ABI_VERSION; }
int fc_last_hip_error(void) { return g_last_hip_error; }

const char* fc_status_string(fc_status s) {
    switch (s) {
        case FC_OK: return "FC_OK";
        case FC_E_NULL: return "FC_E_NULL: a required pointer is NULL";
        case FC_E_ARG: return "FC_E_ARG: argument value outside the supported set, or overlapping buffers";
        case FC_E_SHAPE: return "FC_E_SHAPE: sizes do not divide or exceed the supported limits";
        case FC_E_ALIGN: return "FC_E_ALIGN: a data pointer is not 16-byte aligned (meta: 4-byte)";
        case FC_E_LAUNCH: return "FC_E_LAUNCH: kernel launch failed (see fc_last_hip_error)";
    }
    return "unknown fc_status";
}

fc_status fc_quantize(const uint16_t* x, int64_t n, int bits, int group, fc_qmsg out, hipStream_t stream) {
    if (!valid_bits(bits) || !valid_group(group) || n < 0) return FC_E_ARG;
    if (n % group != 0 || n / 16 > kMaxElems) return FC_E_SHAPE;  // n may hold several ranks' buffers
    if (n == 0) return FC_OK;
    if (!x || !out.codes || !out.meta) return FC_E_NULL;
    if (!aligned(x, 16) || !aligned(out.codes, 16) || !aligned(out.meta, 4)) return FC_E_ALIGN;
    const Range xr = rng(x, 2 * n), cr = rng(out.codes, n * bits / 8), mr = rng(out.meta, 4 * (n / group));
    if (overlap(xr, cr) || overlap(xr, mr) || overlap(cr, mr)) return FC_E_ARG;
    return launched(fc::launch_quantize(fc::QuantizeParams{x, n, bits, group, out.codes, out.meta}, stream));
}

fc_status fc_reduce_shard(const fc_qmsg* in, int R, int64_t L, int n_shards, int bits_in, int bits_out, int group,
                          const fc_qmsg* out, hipStream_t stream) {
    if (R < 1 || R > fc::kMaxRanks || n_shards < 1 || n_shards > fc::kMaxRanks || !valid_bits(bits_in) ||
        !valid_bits(bits_out) || !valid_group(group) || L < 0)
        return FC_E_ARG;
    if (L % group != 0 || L > kMaxElems) return FC_E_SHAPE;
    if (L == 0) return FC_OK;
    if (!in || !out) return FC_E_NULL;
    const int64_t cin = L * bits_in / 8, min_ = 4 * (L / group), cout = L * bits_out / 8;
    for (int i = 0; i < n_shards * R; ++i) {
        if (!in[i].codes || !in[i].meta) return FC_E_NULL;
        if (!aligned(in[i].codes, 16) || !aligned(in[i].meta, 4)) return FC_E_ALIGN;
    }
    for (int s = 0; s < n_shards; ++s) {
        if (!out[s].codes || !out[s].meta) return FC_E_NULL;
        if (!aligned(out[s].codes, 16) || !aligned(out[s].meta, 4)) return FC_E_ALIGN;
    }
    for (int s = 0; s < n_shards; ++s) {
        const Range oc = rng(out[s].codes, cout), om = rng(out[s].meta, min_);
        if (overlap(oc, om)) return FC_E_ARG;
        for (int t = s + 1; t < n_shards; ++t)
            if (overlap(oc, rng(out[t].codes, cout)) || overlap(oc, rng(out[t].meta, min_)) ||
                overlap(om, rng(out[t].codes, cout)) || overlap(om, rng(out[t].meta, min_)))
                return FC_E_ARG;
        for (int i = 0; i < n_shards * R; ++i) {
            const Range ic = rng(in[i].codes, cin), im = rng(in[i].meta, min_);
            if (overlap(oc, ic) || overlap(oc, im) || overlap(om, ic) || overlap(om, im)) return FC_E_ARG;
        }
    }
    // The (shard, rank) pointer table travels as kernel arguments, at most kMaxReduceIn entries per
    // launch: shards are handed to the launcher in groups that fit.
    fc::ReduceParams p;
    const int per_launch = fc::kMaxReduceIn / R;
    for (int s0 = 0; s0 < n_shards; s0 += per_launch) {
        const int ns = (n_shards - s0) < per_launch ? (n_shards - s0) : per_launch;
        for (int i = 0; i < ns * R; ++i) {
            p.in_codes[i] = in[s0 * R + i].codes;
            p.in_meta[i] = in[s0 * R + i].meta;
        }
        for (int i = 0; i < ns; ++i) {
            p.out_codes[i] = out[s0 + i].codes;
            p.out_meta[i] = out[s0 + i].meta;
        }
        p.R = R;
        p.n_shards = ns;
        p.L = L;
        p.bits_in = bits_in;
        p.bits_out = bits_out;
        p.group = group;
        const fc_status st = launched(fc::launch_reduce(p, stream));
        if (st != FC_OK) return st;
    }
    return FC_OK;
}

fc_status fc_reduce_shard_norm(const fc_qmsg* in, int R, int64_t L, int n_shards, int bits_in, int bits_out,
                               int group, const fc_norm* norm, const fc_qmsg* out, hipStream_t stream) {
    if (R < 1 || R > fc::kMaxRanks || n_shards < 1 || n_shards > fc::kMaxRanks || !valid_bits(bits_in) ||
        !valid_bits(bits_out) || !valid_group(group) || L < 0)
        return FC_E_ARG;
    if (!norm) return FC_E_NULL;
    if (!norm->gamma) return FC_E_NULL;
    if (norm->out) return FC_E_ARG;  // the normalized rows go to the quantized messages
    if (!(norm->eps > 0.0f) || norm->eps != norm->eps || norm->eps > 3.0e38f) return FC_E_ARG;
    const int64_t H = norm->hidden;
    if (H <= 0 || H % 8 != 0 || H > kMaxHidden || H % group != 0) return FC_E_SHAPE;
    if (L % group != 0 || L % H != 0 || L > kMaxElems) return FC_E_SHAPE;
    if (L == 0) return FC_OK;
    if (!in || !out) return FC_E_NULL;
    if (!aligned(norm->gamma, 16) || (norm->residual && !aligned(norm->residual, 16)) ||
        (norm->residual_out && !aligned(norm->residual_out, 16)))
        return FC_E_ALIGN;
    const int64_t cin = L * bits_in / 8, min_ = 4 * (L / group), cout = L * bits_out / 8;
    const int64_t nb = 2 * (int64_t)n_shards * L;  // bytes of the shards' residual rows
    for (int i = 0; i < n_shards * R; ++i) {
        if (!in[i].codes || !in[i].meta) return FC_E_NULL;
        if (!aligned(in[i].codes, 16) || !aligned(in[i].meta, 4)) return FC_E_ALIGN;
    }
    for (int s = 0; s < n_shards; ++s) {
        if (!out[s].codes || !out[s].meta) return FC_E_NULL;
        if (!aligned(out[s].codes, 16) || !aligned(out[s].meta, 4)) return FC_E_ALIGN;
    }
    // outputs: the n_shards messages and residual_out; none may overlap another output or any input
    const Range g = rng(norm->gamma, 2 * H);
    const Range ro = norm->residual_out ? rng(norm->residual_out, nb) : Range{0, 0};
    if (norm->residual_out) {
        if (overlap(ro, g)) return FC_E_ARG;
        if (norm->residual && norm->residual != norm->residual_out && overlap(ro, rng(norm->residual, nb)))
            return FC_E_ARG;
    }
    for (int s = 0; s < n_shards; ++s) {
        const Range oc = rng(out[s].codes, cout), om = rng(out[s].meta, min_);
        if (overlap(oc, om) || overlap(oc, g) || overlap(om, g) || overlap(oc, ro) || overlap(om, ro)) return FC_E_ARG;
        if (norm->residual && (overlap(oc, rng(norm->residual, nb)) || overlap(om, rng(norm->residual, nb))))
            return FC_E_ARG;
        for (int t = s + 1; t < n_shards; ++t)
            if (overlap(oc, rng(out[t].codes, cout)) || overlap(oc, rng(out[t].meta, min_)) ||
                overlap(om, rng(out[t].codes, cout)) || overlap(om, rng(out[t].meta, min_)))
                return FC_E_ARG;
    }
    for (int i = 0; i < n_shards * R; ++i) {
        const Range ic = rng(in[i].codes, cin), im = rng(in[i].meta, min_);
        if (overlap(ro, ic) || overlap(ro, im)) return FC_E_ARG;
        for (int s = 0; s < n_shards; ++s) {
            const Range oc = rng(out[s].codes, cout), om = rng(out[s].meta, min_);
            if (overlap(oc, ic) || overlap(oc, im) || overlap(om, ic) || overlap(om, im)) return FC_E_ARG;
        }
    }
    fc::ReduceNormQParams q;
    q.norm = norm_params(norm);
    const int per_launch = fc::kMaxReduceIn / R;
    for (int s0 = 0; s0 < n_shards; s0 += per_launch) {
        const int ns = (n_shards - s0) < per_launch ? (n_shards - s0) : per_launch;
        fc::ReduceParams& p = q.rs;
        for (int i = 0; i < ns * R; ++i) {
            p.in_codes[i] = in[s0 * R + i].codes;
            p.in_meta[i] = in[s0 * R + i].meta;
        }
        for (int i = 0; i < ns; ++i) {
            p.out_codes[i] = out[s0 + i].codes;
            p.out_meta[i] = out[s0 + i].meta;
        }
        p.R = R;
        p.n_shards = ns;
        p.L = L;
        p.bits_in = bits_in;
        p.bits_out = bits_out;
        p.group = group;
        q.norm.residual = norm->residual ? norm->residual + (int64_t)s0 * L : nullptr;
        q.norm.residual_out = norm->residual_out ? norm->residual_out + (int64_t)s0 * L : nullptr;
        const fc_status st = launched(fc::launch_reduce_norm(q, stream));
        if (st != FC_OK) return st;
    }
    return FC_OK;
}

fc_status fc_gather_dequant(const fc_qmsg* shards, int R, int64_t L, int bits, int group, uint16_t* y,
                            const fc_norm* norm, hipStream_t stream) {
    if (R < 1 || R > fc::kMaxRanks || !valid_bits(bits) || !valid_group(group) || L < 0) return FC_E_ARG;
    if (L % group != 0 || (int64_t)R * L > kMaxElems) return FC_E_SHAPE;
    if (!y && !norm) return FC_E_NULL;
    const int64_t n = (int64_t)R * L;
    if (norm) {
        const fc_status st = check_norm(norm, n);
        if (st != FC_OK) return st;
    }
    if (n == 0) return FC_OK;
    if (!shards) return FC_E_NULL;
    const int64_t cb = L * bits / 8, mb = 4 * (L / group);
    for (int s = 0; s < R; ++s) {
        if (!shards[s].codes || !shards[s].meta) return FC_E_NULL;
        if (!aligned(shards[s].codes, 16) || !aligned(shards[s].meta, 4)) return FC_E_ALIGN;
    }
    if (y && !aligned(y, 16)) return FC_E_ALIGN;
    // outputs must not overlap any input
    Range outs[3];
    int nout = 0;
    if (y) outs[nout++] = rng(y, 2 * n);
    if (norm) {
        outs[nout++] = rng(norm->out, 2 * n);
        if (norm->residual_out) outs[nout++] = rng(norm->residual_out, 2 * n);
    }
    for (int o = 0; o < nout; ++o) {
        for (int s = 0; s < R; ++s)
            if (overlap(outs[o], rng(shards[s].codes, cb)) || overlap(outs[o], rng(shards[s].meta, mb))) return FC_E_ARG;
        for (int q = o + 1; q < nout; ++q)
            if (overlap(outs[o], outs[q])) return FC_E_ARG;
        if (norm && o == 0 && y) {
            if (overlap(outs[0], rng(norm->gamma, 2 * norm->hidden))) return FC_E_ARG;
            if (norm->residual && overlap(outs[0], rng(norm->residual, 2 * n))) return FC_E_ARG;
        }
    }
    fc::GatherParams p;
    for (int s = 0; s < fc::kMaxRanks; ++s) {
        p.codes[s] = s < R ? shards[s].codes : nullptr;
        p.meta[s] = s < R ? shards[s].meta : nullptr;
    }
    p.R = R;
    p.L = L;
    p.bits = bits;
    p.group = group;
    p.y = y;
    p.has_norm = norm != nullptr;
    if (norm) p.norm = norm_params(norm);
    return launched(fc::launch_gather(p, stream));
}

fc_status fc_reduce_rmsnorm(const uint16_t* const* parts, int R, int64_t rows, const fc_norm* norm, int max_workgroups,
                            hipStream_t stream) {
    if (R < 1 || R > fc::kMaxRanks || rows < 0 || max_workgroups < 0) return FC_E_ARG;
    if (!norm) return FC_E_NULL;
    if (norm->hidden <= 0 || norm->hidden % 8 != 0 || norm->hidden > kMaxHidden) return FC_E_SHAPE;
    if (rows > kMaxElems / norm->hidden) return FC_E_SHAPE;
    const int64_t n = rows * norm->hidden;
    const fc_status st = check_norm(norm, n);
    if (st != FC_OK) return st;
    if (rows == 0) return FC_OK;
    if (!parts) return FC_E_NULL;
    for (int r = 0; r < R; ++r) {
        if (!parts[r]) return FC_E_NULL;
        if (!aligned(parts[r], 16)) return FC_E_ALIGN;
        const Range pr = rng(parts[r], 2 * n);
        if (overlap(pr, rng(norm->out, 2 * n)) || (norm->residual_out && overlap(pr, rng(norm->residual_out, 2 * n))))
            return FC_E_ARG;
    }
    fc::ReduceNormParams p;
    for (int r = 0; r < fc::kMaxRanks; ++r) p.parts[r] = r < R ? parts[r] : nullptr;
    p.R = R;
    p.rows = rows;
    p.norm = norm_params(norm);
    p.max_workgroups = max_workgroups;
    return launched(fc::launch_reduce_rmsnorm(p, stream));
}

fc_status fc_ll_unpack_reduce(const uint64_t* const* slots, int R, int64_t n, int block_slots, uint32_t epoch,
                              uint16_t* out, uint8_t* stale, uint8_t* done, uint32_t* counters, hipStream_t stream) {
    if (R < 1 || R > fc::kMaxRanks || !valid_block(block_slots) || n < 0) return FC_E_ARG;
    if (n % (2 * block_slots) != 0 || n > kMaxElems) return FC_E_SHAPE;
    if (n == 0) return FC_OK;
    if (!slots || !out || !stale || !done) return FC_E_NULL;
    if (!aligned(out, 16) || (counters && !aligned(counters, 8))) return FC_E_ALIGN;
    const int64_t nblk = n / 2 / block_slots;
    const Range ro = rng(out, 2 * n), rs = rng(stale, (int64_t)R * nblk), rd = rng(done, nblk), rc = rng(counters, counters ? 4 * FC_COUNTER_WORDS : 0);
    if (overlap(ro, rs) || overlap(ro, rd) || overlap(ro, rc) || overlap(rs, rd) || overlap(rs, rc) || overlap(rd, rc))
        return FC_E_ARG;
    for (int r = 0; r < R; ++r) {
        if (!slots[r]) return FC_E_NULL;
        if (!aligned(slots[r], 16)) return FC_E_ALIGN;
        const Range sr = rng(slots[r], 4 * n);
        if (overlap(sr, ro) || overlap(sr, rs) || overlap(sr, rd) || overlap(sr, rc)) return FC_E_ARG;
    }
    fc::LLParams p;
    for (int r = 0; r < fc::kMaxRanks; ++r) p.slots[r] = r < R ? slots[r] : nullptr;
    p.R = R;
    p.n = n;
    p.block_slots = block_slots;
    p.epoch = epoch;
    p.out = out;
    p.stale = stale;
    p.done = done;
    p.counters = counters;
    return launched(fc::launch_ll_unpack(p, stream));
}

fc_status fc_ll_gather(const uint64_t* const* slots, int R, int64_t nwords, int block_slots, uint32_t epoch,
                       uint32_t* const* out, uint8_t* stale, uint8_t* done, uint32_t* counters, hipStream_t stream) {
    if (R < 1 || R > fc::kMaxRanks || !valid_block(block_slots) || nwords < 0) return FC_E_ARG;
    if (nwords % block_slots != 0 || nwords > kMaxElems) return FC_E_SHAPE;
    if (nwords == 0) return FC_OK;
    if (!slots || !out || !stale || !done) return FC_E_NULL;
    if ((counters && !aligned(counters, 8))) return FC_E_ALIGN;
    const int64_t nblk = nwords / block_slots;
    const Range rs = rng(stale, (int64_t)R * nblk), rd = rng(done, (int64_t)R * nblk), rc = rng(counters, counters ? 4 * FC_COUNTER_WORDS : 0);
    if (overlap(rs, rd) || overlap(rs, rc) || overlap(rd, rc)) return FC_E_ARG;
    for (int r = 0; r < R; ++r) {
        if (!slots[r] || !out[r]) return FC_E_NULL;
        if (!aligned(slots[r], 16) || !aligned(out[r], 8)) return FC_E_ALIGN;
    }
    for (int r = 0; r < R; ++r) {
        const Range ro = rng(out[r], 4 * nwords);
        if (overlap(ro, rs) || overlap(ro, rd) || overlap(ro, rc)) return FC_E_ARG;
        for (int q = 0; q < R; ++q) {
            const Range sq = rng(slots[q], 8 * nwords);
            if (overlap(ro, sq)) return FC_E_ARG;
            if (q > r && overlap(ro, rng(out[q], 4 * nwords))) return FC_E_ARG;
            if (r == 0 && (overlap(sq, rs) || overlap(sq, rd) || overlap(sq, rc))) return FC_E_ARG;
        }
    }
    fc::LLGatherParams p;
    for (int r = 0; r < fc::kMaxRanks; ++r) {
        p.slots[r] = r < R ? slots[r] : nullptr;
        p.out[r] = r < R ? out[r] : nullptr;
    }
    p.R = R;
    p.nwords = nwords;
    p.block_slots = block_slots;
    p.epoch = epoch;
    p.stale = stale;
    p.done = done;
    p.counters = counters;
    return launched(fc::launch_ll_gather(p, stream));
}

fc_status fc_ll_pack(const uint16_t* const* x, int R, int64_t n, int block_slots, uint32_t epoch,
                     const int32_t* const* block_order, int pace, uint64_t* const* slots, hipStream_t stream) {
    if (R < 1 || R > fc::kMaxRanks || !valid_block(block_slots) || n < 0 || pace < 0 || pace > kMaxPace)
        return FC_E_ARG;
    if (n % (2 * block_slots) != 0 || n > kMaxElems) return FC_E_SHAPE;
    if (n == 0) return FC_OK;
    if (!x || !slots) return FC_E_NULL;
    const int64_t nblk = n / 2 / block_slots;
    for (int r = 0; r < R; ++r) {
        if (!x[r] || !slots[r]) return FC_E_NULL;
        const int32_t* o = block_order ? block_order[r] : nullptr;
        if (!aligned(x[r], 16) || !aligned(slots[r], 16) || (o && !aligned(o, 4))) return FC_E_ALIGN;
    }
    for (int r = 0; r < R; ++r) {  // a rank's slots overlap no input of any rank and no other rank's slots
        const Range sr = rng(slots[r], 4 * n);
        for (int q = 0; q < R; ++q) {
            const int32_t* o = block_order ? block_order[q] : nullptr;
            if (overlap(sr, rng(x[q], 2 * n)) || (o && overlap(sr, rng(o, 4 * nblk)))) return FC_E_ARG;
            if (q > r && overlap(sr, rng(slots[q], 4 * n))) return FC_E_ARG;
        }
    }
    fc::PackParams p;
    for (int r = 0; r < fc::kMaxRanks; ++r) {
        p.x[r] = r < R ? x[r] : nullptr;
        p.order[r] = r < R && block_order ? block_order[r] : nullptr;
        p.slots[r] = r < R ? slots[r] : nullptr;
    }
    p.R = R;
    p.n = n;
    p.block_slots = block_slots;
    p.epoch = epoch;
    p.pace = pace;
    return launched(fc::launch_ll_pack(p, stream));
}

fc_status fc_ll_poll_unpack_reduce(const uint64_t* const* slots, int R, int64_t n, int block_slots, uint32_t epoch,
                                   int max_polls, int max_workgroups, uint16_t* out, uint8_t* stale, uint8_t* done,
                                   uint32_t* counters, hipStream_t stream) {
    if (R < 1 || R > fc::kMaxRanks || !valid_block(block_slots) || n < 0) return FC_E_ARG;
    if (max_polls < 0 || max_polls > kMaxPolls || max_workgroups < 0) return FC_E_ARG;
    if (n % (2 * block_slots) != 0 || n > kMaxElems) return FC_E_SHAPE;
    if (n == 0) return FC_OK;
    if (!slots || !out || !stale || !done) return FC_E_NULL;
    if (!aligned(out, 16) || (counters && !aligned(counters, 8))) return FC_E_ALIGN;
    const int64_t nblk = n / 2 / block_slots;
    const Range ro = rng(out, 2 * n), rs = rng(stale, (int64_t)R * nblk), rd = rng(done, nblk), rc = rng(counters, counters ? 4 * FC_COUNTER_WORDS : 0);
    if (overlap(ro, rs) || overlap(ro, rd) || overlap(ro, rc) || overlap(rs, rd) || overlap(rs, rc) || overlap(rd, rc))
        return FC_E_ARG;
    for (int r = 0; r < R; ++r) {
        if (!slots[r]) return FC_E_NULL;
        if (!aligned(slots[r], 16)) return FC_E_ALIGN;
        const Range sr = rng(slots[r], 4 * n);
        if (overlap(sr, ro) || overlap(sr, rs) || overlap(sr, rd) || overlap(sr, rc)) return FC_E_ARG;
    }
    fc::LLParams p;
    for (int r = 0; r < fc::kMaxRanks; ++r) p.slots[r] = r < R ? slots[r] : nullptr;
    p.R = R;
    p.n = n;
    p.block_slots = block_slots;
    p.epoch = epoch;
    p.out = out;
    p.stale = stale;
    p.done = done;
    p.counters = counters;
    return launched(fc::launch_ll_poll(p, fc::PollParams{max_polls, max_workgroups}, stream));
}

fc_status fc_flag_unpack_reduce(const uint16_t* const* payload, const uint32_t* const* flags, int R, int64_t n,
                                int block_elems, uint32_t epoch, int max_polls, int max_workgroups, uint16_t* out,
                                uint8_t* stale, uint8_t* done, uint32_t* counters, hipStream_t stream) {
    const int lb = log2_flag_block(block_elems);
    if (R < 1 || R > fc::kMaxRanks || lb < 0 || n < 0) return FC_E_ARG;
    if (max_polls < 0 || max_polls > kMaxPolls || max_workgroups < 0) return FC_E_ARG;
    if (n % block_elems != 0 || n > kMaxElems) return FC_E_SHAPE;
    if (n == 0) return FC_OK;
    if (!payload || !flags || !out || !stale || !done) return FC_E_NULL;
    if (!aligned(out, 16) || (counters && !aligned(counters, 8))) return FC_E_ALIGN;
    const int64_t nblk = n / block_elems;
    const Range ro = rng(out, 2 * n), rs = rng(stale, (int64_t)R * nblk), rd = rng(done, nblk), rc = rng(counters, counters ? 4 * FC_COUNTER_WORDS : 0);
    if (overlap(ro, rs) || overlap(ro, rd) || overlap(ro, rc) || overlap(rs, rd) || overlap(rs, rc) || overlap(rd, rc))
        return FC_E_ARG;
    for (int r = 0; r < R; ++r) {
        if (!payload[r] || !flags[r]) return FC_E_NULL;
        if (!aligned(payload[r], 16) || !aligned(flags[r], 4)) return FC_E_ALIGN;
        for (const Range in : {rng(payload[r], 2 * n), rng(flags[r], 4 * nblk)})
            if (overlap(in, ro) || overlap(in, rs) || overlap(in, rd) || overlap(in, rc)) return FC_E_ARG;
    }
    fc::FlagParams p;
    for (int r = 0; r < fc::kMaxRanks; ++r) {
        p.payload[r] = r < R ? payload[r] : nullptr;
        p.flags[r] = r < R ? flags[r] : nullptr;
    }
    p.R = R;
    p.n = n;
    p.log2_block = lb;
    p.epoch = epoch;
    p.out = out;
    p.stale = stale;
    p.done = done;
    p.counters = counters;
    p.poll = fc::PollParams{max_polls, max_workgroups};
    return launched(fc::launch_flag_unpack(p, stream));
}

fc_status fc_flag_pack(const uint16_t* const* x, int R, int64_t n, int block_elems, uint32_t epoch,
                       const int32_t* const* block_order, int pace, uint16_t* const* payload, uint32_t* const* flags,
                       hipStream_t stream) {
    const int lb = log2_flag_block(block_elems);
    if (R < 1 || R > fc::kMaxRanks || lb < 0 || n < 0 || pace < 0 || pace > kMaxPace) return FC_E_ARG;
    if (n % block_elems != 0 || n > kMaxElems) return FC_E_SHAPE;
    if (n == 0) return FC_OK;
    if (!x || !payload || !flags) return FC_E_NULL;
    const int64_t nblk = n / block_elems;
    for (int r = 0; r < R; ++r) {
        if (!x[r] || !payload[r] || !flags[r]) return FC_E_NULL;
        const int32_t* o = block_order ? block_order[r] : nullptr;
        if (!aligned(x[r], 16) || !aligned(payload[r], 16) || !aligned(flags[r], 4) || (o && !aligned(o, 4)))
            return FC_E_ALIGN;
    }
    for (int r = 0; r < R; ++r) {  // outputs overlap no input of any rank and no other output
        const Range rp = rng(payload[r], 2 * n), rf = rng(flags[r], 4 * nblk);
        if (overlap(rp, rf)) return FC_E_ARG;
        for (int q = 0; q < R; ++q) {
            const int32_t* o = block_order ? block_order[q] : nullptr;
            for (const Range out : {rp, rf}) {
                if (overlap(out, rng(x[q], 2 * n)) || (o && overlap(out, rng(o, 4 * nblk)))) return FC_E_ARG;
                if (q > r && (overlap(out, rng(payload[q], 2 * n)) || overlap(out, rng(flags[q], 4 * nblk))))
                    return FC_E_ARG;
            }
        }
    }
    fc::FlagPackParams p;
    for (int r = 0; r < fc::kMaxRanks; ++r) {
        p.x[r] = r < R ? x[r] : nullptr;
        p.order[r] = r < R && block_order ? block_order[r] : nullptr;
        p.payload[r] = r < R ? payload[r] : nullptr;
        p.flags[r] = r < R ? flags[r] : nullptr;
    }
    p.R = R;
    p.n = n;
    p.log2_block = lb;
    p.epoch = epoch;
    p.pace = pace;
    return launched(fc::launch_flag_pack(p, stream));
}

fc_status fc_bandwidth_probe(const void* src, void* dst, int64_t bytes, int mode, hipStream_t stream) {
    if (mode < 0 || mode > 2 || bytes < 0) return FC_E_ARG;
    if (bytes % 16 != 0 || bytes > (int64_t(1) << 40)) return FC_E_SHAPE;
    if (bytes == 0) return FC_OK;
    if ((mode != 2 && !src) || !dst) return FC_E_NULL;  // dst: the copy's target, the sink, or the written range
    if ((src && !aligned(src, 16)) || !aligned(dst, mode == 1 ? 4 : 16)) return FC_E_ALIGN;
    if (mode == 0 && overlap(rng(src, bytes), rng(dst, bytes))) return FC_E_ARG;
    if (mode == 1 && overlap(rng(src, bytes), rng(dst, 4))) return FC_E_ARG;
    return launched(fc::launch_bandwidth_probe(src, dst, bytes, mode, stream));
}

fc_status fc_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
    if (bytes < 0) return FC_E_ARG;
    if (bytes % 16 != 0 || bytes > (int64_t(1) << 40)) return FC_E_SHAPE;
    if (bytes == 0) return FC_OK;
    if (!src || !dst) return FC_E_NULL;
    if (!aligned(src, 16) || !aligned(dst, 16)) return FC_E_ALIGN;
    if (overlap(rng(src, bytes), rng(dst, bytes))) return FC_E_ARG;
    return launched(fc::launch_copy(src, dst, bytes, stream));
}

}  // extern "C"
