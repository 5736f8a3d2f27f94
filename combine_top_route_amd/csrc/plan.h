// Launch plan and workspace layout shared by the host API and the kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "ubep.h"

namespace ubep {

// Implemented limits (checked by ubep_check_shape).
constexpr int kMaxK = 32;
constexpr int kMaxR = 1024;
constexpr int kMaxE = 8192;
constexpr int kMaxC = 256;
constexpr int kGateMaxE = 1024;
constexpr int kGateMaxGroups = 64;
constexpr int kExpertMaxE = 1024;        // experts of ubep_expert_linear
constexpr int64_t kExpertMaxRowTiles = 65535;   // row tiles (grid.y) of ubep_expert_linear

// Layout kernel: 8 waves per workgroup, tiles of whole tokens with at most
// kTileRowsMax rows.  A workgroup ranks its tile's rows one 64-row step after
// another, so tiles are also kept small enough for about kTileTarget of them
// (the ranking then runs on that many CUs at once), but not below
// kTileRowsMin rows.
constexpr int kLayoutThreads = 512;
constexpr int kLayoutWaves = 8;
constexpr int64_t kTileRowsMax = 4096;
constexpr int64_t kTileTarget = 128;
constexpr int64_t kTileRowsMin = 256;
constexpr int64_t kLdsBytesPerCu = 160 * 1024;

// Workspace header: 32-bit counters, each on its own 128-byte line.
constexpr int kHdrStatus = 0;          // device status word (ubep_status)
constexpr int kHdrLayoutTicket = 32;   // tile ticket of the layout scan
constexpr int kHdrFusedTicket = 64;    // task ticket of the chunk pipeline
constexpr int kHdrFusedDone = 96;      // workgroups finished in the chunk pipeline
constexpr int kHdrLayoutDone = 128;    // workgroups finished in the layout
constexpr int kHdrLayoutEpoch = 160;   // layout calls completed (tags look-back state)
constexpr int kHdrRoleTicket = 192;    // role ticket of the fused layout + dispatch kernel
constexpr int kHdrPosReady = 224;      // layout workers whose positions are stored
constexpr int kHdrCombineTicket = 256; // block ticket of the combine's later workgroups
constexpr int kHdrDispatchTicket = 288; // block ticket of the dispatch's later workgroups
constexpr int kHdrFusedBlockTicket = 320; // block ticket of the fused launch's later workgroups
constexpr int kHdrSentTicket = 352;    // task ticket of the sentinel-readiness pipeline
constexpr int kHdrSentDone = 384;      // workgroups finished in the sentinel-readiness pipeline
constexpr int kHdrSentGiveUp = 416;    // set once a sentinel wait has expired: later waits give up
constexpr int kHdrFusedGiveUp = 448;   // set once a chunk-flag wait has expired: later waits give up
constexpr int kHdrGateLayoutDone = 480; // workgroups finished in the layout from gate counts
constexpr size_t kHdrBytes = 2048;
// Readiness sentinel of the sentinel-polling pipeline: every 32-bit word of a
// receive row's first 16-byte unit while the row is empty (two bf16 NaNs).
constexpr uint32_t kRowSentinelWord = 0xFFFFFFFFu;
constexpr int kFlagStride = 32;        // uint32 per chunk ready flag (128 bytes)

// Look-back state word (64 bits): the layout call's epoch in the high half;
// in the low half a 2-bit flag above a 30-bit row count (T*k < 2^30).  A word
// whose epoch is not the current call's is "not published yet", so the state
// never needs clearing between calls.
constexpr uint32_t kCountMask = (1u << 30) - 1u;
constexpr uint32_t kFlagAggregate = 1u << 30;   // this tile's own count is known
constexpr uint32_t kFlagInclusive = 2u << 30;   // count of this and all earlier tiles
constexpr int kLookbackWindow = 32;              // predecessor states read per round
constexpr int kMaxTilesPerGroup = 256;           // tiles one layout workgroup may claim
// Gather mode (few tiles): every worker sums all tiles' published counts
// instead of looking back; a worker then claims at most kGatherMaxMine tiles.
constexpr int64_t kGatherMaxWords = 16384;       // n_tiles * K
constexpr int64_t kGatherMaxTiles = 512;
constexpr int kGatherMaxMine = 8;
constexpr int kGatherBurst = 8;                  // state words a thread loads at once
constexpr int64_t kMaxStateWords = (int64_t)1 << 26;                   // look-back state cap
// Per-device scratch array of the allocation-free layout (ubep_layout_noalloc):
// the largest workspace it serves.
constexpr size_t kScratchBytes = (size_t)8 << 20;
constexpr int kScratchMaxDevices = 64;

struct Plan {
    int64_t T, H;
    int32_t E, k, R, C;
    int64_t rows;          // T*k
    int32_t epr;           // experts per rank
    uint32_t epr_magic;    // ceil(2^32 / epr), 0 when epr == 1: rank = umulhi(e, magic)
    int64_t tps;           // tokens per source rank
    int64_t tpc;           // tokens per chunk
    int64_t tile_tokens;   // tokens per layout tile; divides tps and tpc
    int64_t tile_rows;     // tile_tokens * k
    int64_t n_tiles;
    int32_t dbits;         // bits to hold a rank id (0..R-1)
    int32_t ebits;         // bits to hold an expert id (0..E-1)
    int32_t gather;        // 1: prefixes and totals by gathering all tiles' counts
    // workspace byte offsets
    int32_t slots;         // look-back digits per tile: R ranks, then E experts
    size_t off_state;      // uint64 [n_tiles_ws][R+E]  look-back state
    size_t off_excl;       // int32  [n_tiles_ws][K]    rows with key q in earlier tiles (sized for K = E)
    size_t off_wbase;      // int32  [n_tiles_ws][8][K] rows with key q in earlier waves of the tile
    size_t off_flags;      // uint32 [C][kFlagStride] chunk ready flags
    size_t ws_bytes;
    size_t off_order;      // int32  [C] chunk order computed on the device (LPT policy)
    size_t off_gate_rank;  // int32  [n_tiles_ws][R] rows per (tile, rank) counted by the gate
    size_t off_gate_expert; // int32 [n_tiles_ws][E] rows per (tile, expert) counted by the gate
    // Position keys (last, so that the fields the rank-order kernels read keep
    // their places).  Rank order: rows sort by (rank, token, slot), one key
    // per rank.  Expert order: rows sort by (expert, token, slot), one key per
    // expert (a rank's experts are consecutive, so its region is still one
    // run).  key(e) = rank_of(e, key_magic).
    int32_t order;         // 0: rank order, 1: expert order
    int32_t K;             // keys: R or E
    uint32_t key_magic;    // epr_magic (rank order) or 0 (expert order: key = e)
    int32_t kbits;         // bits to hold a key
    int32_t kcol;          // state digit of key 0: 0 (rank digits) or R (expert digits)
    int64_t n_tiles_ws;    // tiles the workspace arrays are sized for (>= n_tiles)
};

// Host: fill `p` for a shape that passed validation; order 0 (rank order)
// or 1 (expert order); spread: the tiling with about kTileTarget tiles, else
// the one with the largest tiles.  The workspace layout depends on neither
// (it is the spread tiling's) unless ws_spread is false, when it is laid out
// for the tiling in use alone.
void make_plan(const ubep_shape& s, Plan* p, int order = 0, bool spread = true, bool ws_spread = true);

}  // namespace ubep
