// moe_layout.h -- device data layout shared by the repack kernels, the compute kernels and the host
// code of the MI355X MoE decode library.
//
// Expert weights are repacked once (moe_decode_set_layer) from their canonical row-major form into
// "K-major lane tiles": the 16-byte unit (one MX block: 32 E2M1 codes) a lane loads at step s of
// its loop sits right after the units its 63 neighbours load at the same step, so every wave-wide
// load instruction reads 1 KiB of contiguous HBM.  The repack only permutes 16-byte units and
// scale bytes; no value changes.  The router stays row-major (one wave reads one 5 KiB row).
//
//   router  [E][H] bf16, canonical.
//   w13     [E+S][I/16 tiles][GW waves][BPL steps][64 lanes][16 B]
//             lane l: tile row r = l/2 (r < 16: gate row 16*tile + r, else up row I + 16*tile + r-16),
//             MX block (w*BPL + step)*2 + l%2 of that row (GW*BPL*2 = H/32).
//   w13_s   [E+S][I/16][GW][64 lanes][BPL bytes]   the scales of those BPL blocks.
//   w2      [E+S][H/R tiles][ITERS][64 lanes][16 B]   R = 64/KSUB rows per tile,
//             lane l: row R*tile + l/KSUB, MX block it*KSUB + l%KSUB (KSUB*ITERS = I/32).
//   w2_s    [E+S][H/R][ITERS][64 lanes]            one scale byte per unit above.
//
// Per-call intermediate data lives in the handle's workspace, indexed by "pair" p = t*(k+S) + r:
// token t, rank r < k (routed) or r = k (the shared expert).
#pragma once
#ifndef __HIPCC_RTC__
#include <stdint.h>
#endif

namespace moe {

constexpr int kWave = 64;
constexpr int kBlock = 32;          // K elements per MX block (one E8M0 scale) = one 16-byte unit
constexpr int kMaxTokens = 4;
constexpr int kMaxTopK = 8;
constexpr int kMaxExperts = 512;
constexpr int kMaxSlots = kMaxTokens * kMaxTopK;   // distinct routed experts of one call
constexpr int kMaxPairs = kMaxTokens * (kMaxTopK + 1);
constexpr int kGuRows = 32;         // rows per gate/up tile: 16 gate + 16 up
constexpr int kGuOut = 16;          // h outputs per gate/up tile
constexpr int kMaxWaves = 5;        // waves per workgroup of the router / gate/up kernels
// Token counts from which h is requantised once per layer by its own kernel (below, every down
// workgroup requantises all h rows itself: at 4 tokens, 36 rows per workgroup, that measured
// 28.7 us for the down kernel against 11.2 us plus 1.4 us for the requantisation kernel).
constexpr int kKqMinT = 3;
// Token counts up to which every routed gate/up workgroup takes the top-k itself (VALU form: 3,
// matrix-core form: 2); above, the last router workgroup takes it once, behind an arrival ticket.
// Measured on the 42-layer stack, us/layer: VALU form, top-k in gate/up at 3 tokens 37.8 against
// 38.9 with the ticket, at 4 tokens 47.5 against 44.7 (1,536 workgroups each redoing four top-k's
// cost more than the ticket's tail); matrix-core form at 3 tokens 41.6 against 39.0 (its 76-VGPR
// workgroups, four per CU, run the 3-token grid in two rounds, each paying the top-k).
constexpr int gu_route_max_t(bool mfma) { return mfma ? 2 : 3; }
constexpr int kDownGrid = 256;      // workgroups of the down kernel: one per compute unit (H % 256 == 0)

// Work list of the routed experts of one call, built identically by every workgroup of the
// gate/up kernel from the router logits (workgroup 0 also stores it for the down kernel).
struct SlotTable {
    int n;                            // number of distinct routed experts
    int pad[3];
    int expert[kMaxSlots];            // expert index
    int ntok[kMaxSlots];              // tokens routed to it
    int tok[kMaxSlots][kMaxTokens];   // which tokens, ascending
    int rank[kMaxSlots][kMaxTokens];  // its rank in each of those tokens' top-k
    float w[kMaxSlots][kMaxTokens];   // routing weight for each of those tokens
};

struct Shape {
    int H, E, k, S, I;
    int NB() const { return H / kBlock; }                    // MX blocks along H
    int bpl() const { return NB() % 16 == 0 ? 8 : 4; }       // gate/up blocks per lane and wave
    int gw() const { return NB() / (2 * bpl()); }            // waves of the router / gate/up kernels
    int gu_tiles() const { return I / kGuOut; }
    int NI() const { return I / kBlock; }                    // MX blocks along I
    int ksub() const { return NI() % 8 == 0 ? 8 : NI() % 4 == 0 ? 4 : 2; }
    int iters() const { return NI() / ksub(); }
    int down_rows() const { return kWave / ksub(); }
    int pairs(int T) const { return T * (k + S); }
    uint64_t router_bytes() const { return (uint64_t)E * H * 2; }
    uint64_t w13_bytes_per_expert() const { return (uint64_t)I * H; }          // 2I x H/2
    uint64_t w13s_bytes_per_expert() const { return (uint64_t)2 * I * H / 32; }
    uint64_t w2_bytes_per_expert() const { return (uint64_t)H * I / 2; }
    uint64_t w2s_bytes_per_expert() const { return (uint64_t)H * I / 32; }
};

}  // namespace moe
