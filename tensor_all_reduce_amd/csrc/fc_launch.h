// fc_launch.h -- launch parameters passed from the validating C-ABI layer to the kernel launchers.
// Internal to libfc.so.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace fc {

constexpr int kMaxRanks = 16;
constexpr int kMaxReduceIn = 128;  // (shard, rank) message pointers per reduce launch (kernel-argument table)

struct QuantizeParams {
    const uint16_t* x;
    int64_t n;
    int bits, group;
    uint8_t* codes;
    uint32_t* meta;
};

struct ReduceParams {
    const uint8_t* in_codes[kMaxReduceIn];  // [shard * R + rank]
    const uint32_t* in_meta[kMaxReduceIn];
    uint8_t* out_codes[kMaxRanks];          // [shard]
    uint32_t* out_meta[kMaxRanks];
    int R, n_shards;
    int64_t L;
    int bits_in, bits_out, group;
};

struct NormParams {
    const uint16_t* residual;
    const uint16_t* gamma;
    float eps;
    int64_t hidden;
    uint16_t* out;
    uint16_t* residual_out;
};

struct GatherParams {
    const uint8_t* codes[kMaxRanks];  // [shard]
    const uint32_t* meta[kMaxRanks];
    int R;
    int64_t L;
    int bits, group;
    uint16_t* y;     // plain output or nullptr
    bool has_norm;
    NormParams norm;
};

struct ReduceNormParams {
    const uint16_t* parts[kMaxRanks];
    int R;
    int64_t rows;
    NormParams norm;
    int max_workgroups;
};

struct LLParams {
    const uint64_t* slots[kMaxRanks];
    int R;
    int64_t n;
    int block_slots;
    uint32_t epoch;
    uint16_t* out;
    uint8_t* stale;
    uint8_t* done;
    uint32_t* counters;
};

struct LLGatherParams {
    const uint64_t* slots[kMaxRanks];
    uint32_t* out[kMaxRanks];
    int R;
    int64_t nwords;  // per rank
    int block_slots;
    uint32_t epoch;
    uint8_t* stale;  // [R][nblk]
    uint8_t* done;   // [R][nblk]
    uint32_t* counters;
};

// Sender emulation of R peers writing at the same time (one launch, one grid row per rank).
struct PackParams {
    const uint16_t* x[kMaxRanks];
    const int32_t* order[kMaxRanks];  // entries may be null (ascending)
    uint64_t* slots[kMaxRanks];
    int R;
    int64_t n;
    int block_slots;
    uint32_t epoch;
    int pace;
};

// Receivers that may run while the senders write: bounded re-reads, optional cap on the grid.
struct PollParams {
    int max_polls;      // re-reads of a stale tile, 0 = one look
    int max_workgroups; // 0 = one tile per wavefront
};

struct FlagParams {
    const uint16_t* payload[kMaxRanks];
    const uint32_t* flags[kMaxRanks];
    int R;
    int64_t n;
    int log2_block;  // block of 2^log2_block elements, 9..16
    uint32_t epoch;
    uint16_t* out;
    uint8_t* stale;  // [R][nblk]
    uint8_t* done;   // [nblk]
    uint32_t* counters;
    PollParams poll;
};

struct FlagPackParams {
    const uint16_t* x[kMaxRanks];
    const int32_t* order[kMaxRanks];  // entries may be null (ascending)
    uint16_t* payload[kMaxRanks];
    uint32_t* flags[kMaxRanks];
    int R;
    int64_t n;
    int log2_block;
    uint32_t epoch;
    int pace;
};

// Reduce-scatter receive side with the norm before the all-gather: rs as for launch_reduce; norm's
// residual / residual_out hold the rows of rs's shards in order (shard i at i*L); norm.out is unused.
struct ReduceNormQParams {
    ReduceParams rs;
    NormParams norm;
};

hipError_t launch_quantize(const QuantizeParams& p, hipStream_t s);
hipError_t launch_reduce_norm(const ReduceNormQParams& p, hipStream_t s);
hipError_t launch_reduce(const ReduceParams& p, hipStream_t s);
hipError_t launch_gather(const GatherParams& p, hipStream_t s);
hipError_t launch_reduce_rmsnorm(const ReduceNormParams& p, hipStream_t s);
hipError_t launch_ll_unpack(const LLParams& p, hipStream_t s);
hipError_t launch_ll_pack(const PackParams& p, hipStream_t s);
hipError_t launch_ll_gather(const LLGatherParams& p, hipStream_t s);
hipError_t launch_ll_poll(const LLParams& p, const PollParams& q, hipStream_t s);
hipError_t launch_flag_unpack(const FlagParams& p, hipStream_t s);
hipError_t launch_flag_pack(const FlagPackParams& p, hipStream_t s);
hipError_t launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t s);
hipError_t launch_bandwidth_probe(const void* src, void* dst, int64_t bytes, int mode, hipStream_t s);

}  // namespace fc
