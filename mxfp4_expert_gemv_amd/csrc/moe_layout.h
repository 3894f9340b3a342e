// moe_layout.h -- device data layout shared by the repack kernels, the compute kernels and the host
// code of the MI355X MoE decode library.
//
// All weight tensors are repacked once (moe_decode_set_layer) from their canonical row-major form
// into "K-major lane tiles": the 16-byte unit a lane loads at step s of its loop sits right after
// the units its 63 neighbours load at the same step, so every wave-wide load instruction reads
// 1 KiB of contiguous HBM.  A unit is one MX block (32 E2M1 codes, 16 bytes) or 8 bf16 router
// weights.  The repack only permutes 16-byte units and scale bytes; no value changes.
//
//   router  [RT = ceil(E/64)][H/8][64 lanes][8 bf16]    lane = row within a 64-row tile
//                                                       (rows >= E are zero)
//   w13     [E+S][I/32][H/32][64 lanes][16 B]           lane < 32: gate row 32*tile + lane,
//                                                       lane >= 32: up row I + 32*tile + lane - 32
//   w13_s   [E+S][I/32][H/256][64 lanes][8 B]           the 8 block scales of the 8 consecutive
//                                                       MX blocks one lane reads per wave slice
//   w2      [E+S][H/R][I/(32*KSUB)][64 lanes][16 B]     R = 64/KSUB rows per tile, lane -> row
//                                                       R*tile + lane/KSUB, MX block
//                                                       it*KSUB + lane%KSUB
//   w2_s    [E+S][H/R][I/(32*KSUB)][64 lanes]           one scale byte per unit above
#pragma once
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;
constexpr int kBlock = 32;          // K elements per MX block (one E8M0 scale)
constexpr int kMaxTokens = 4;
constexpr int kMaxTopK = 8;
constexpr int kMaxSlots = kMaxTokens * kMaxTopK + 1;  // distinct routed experts + shared

// router
constexpr int kRouterRows = 64;     // rows per tile (one per lane)
constexpr int kRouterUnitElems = 8; // bf16 per 16-byte unit
constexpr int kRouterUnitsPerWave = 8;
constexpr int kRouterWaves = 4;
constexpr int kRouterSlice = kRouterWaves * kRouterUnitsPerWave * kRouterUnitElems;  // 256 K per WG

// gate/up
constexpr int kGuHalf = 32;         // h outputs per tile (32 gate + 32 up rows)
constexpr int kGuBlocksPerWave = 8; // MX blocks (256 K elements) per wave
constexpr int kGuSlice = kGuBlocksPerWave * kBlock;  // 256

// Work list built by the router's finishing workgroup: the distinct experts of this call.
struct SlotTable {
    int n;                           // number of slots in use
    int pad[3];
    int expert[kMaxSlots];           // expert index (E = the shared expert)
    int ntok[kMaxSlots];             // tokens routed to it
    int tok[kMaxSlots][kMaxTokens];  // which tokens, ascending
    float w[kMaxSlots][kMaxTokens];  // routing weight of each of those tokens (1 for shared)
};

struct Shape {
    int H, E, k, S, I;
    int RT() const { return (E + kRouterRows - 1) / kRouterRows; }
    int down_ksub() const { return (I / kBlock) % 4 == 0 ? 4 : 2; }
    int down_rows() const { return kWave / down_ksub(); }
    int down_iters() const { return I / kBlock / down_ksub(); }
    // bytes of each repacked tensor for one layer
    uint64_t router_bytes() const { return (uint64_t)RT() * kRouterRows * H * 2; }
    uint64_t w13_bytes_per_expert() const { return (uint64_t)I * H; }          // 2I x H/2
    uint64_t w13s_bytes_per_expert() const { return (uint64_t)2 * I * H / 32; }
    uint64_t w2_bytes_per_expert() const { return (uint64_t)H * I / 2; }
    uint64_t w2s_bytes_per_expert() const { return (uint64_t)H * I / 32; }
};

}  // namespace moe
