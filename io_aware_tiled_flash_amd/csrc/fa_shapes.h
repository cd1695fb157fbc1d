// Host-visible description of the kernels: element types, tile sizes, the
// parameter blocks the launches take and the kernel plan. Plain C++ with no
// HIP dependency, so the argument validation that fills these blocks can be
// built and tested on the host alone.
#pragma once

#include <stdint.h>

namespace fa {

enum { kDtypeF32 = 0, kDtypeF16 = 1, kDtypeBF16 = 2 };

// Tiles. The fast bf16/f16 forward streams keys in blocks of kFastBC with 32
// query rows per wave; the generic forward uses kGenericBR x kGenericBC tiles;
// both backward kernels work on blocks of kBwdRows rows (queries or keys).
constexpr int kFastBC = 64;
constexpr int kGenericBR = 128;
constexpr int kGenericBC = 64;
constexpr int kBwdRows = 128;
// Size of the static device scratch of the allocation-free backward: the two
// fp32 per-row arrays of 4M rows (B*H*S with S rounded up to kBwdRows).
constexpr int64_t kBwdScratchBytes = (int64_t)32 << 20;

// ---- Mask segments of a block walk (constexpr: usable in kernels and on the host) ----
//
// The kernels walk their blocks in three segments: [partially visible][fully
// visible][partially visible], where only the end segments carry mask code.
// The functions below give the fully visible run in closed form. Any run of
// fully visible blocks is correct to use (the masked step is exact on a fully
// visible block too); these return the run the mask geometry makes contiguous.

constexpr int cmin(int a, int b) { return a < b ? a : b; }
constexpr int cmax(int a, int b) { return a > b ? a : b; }
// a / b rounded towards -inf / +inf, for b > 0 and any sign of a
constexpr int floor_div(int a, int b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }
constexpr int ceil_div(int a, int b) { return a >= 0 ? (a + b - 1) / b : -((-a) / b); }

struct StepRange {
  int lo, hi;   // steps [lo, hi)
};

// ---- LDS layouts of the bf16/f16 tiles ----
//
// 16-byte chunk swizzle of the K layout: logical chunk c of a row sits at
// c ^ k_swz(row). LDS serves 256 bytes a clock from 64 four-byte banks, so a
// 16-byte read serves 16 lanes a cycle and an 8-byte read 32. The tile is
// read two ways:
//  * rows (an MFMA operand over d): 16 consecutive rows, one logical chunk,
//    in a cycle -- the 16 rows must land in different banks;
//  * transposed (ds_read_b64_tr_b16): 4 consecutive rows x logical chunks
//    4 dt .. 4 dt + 3 in a cycle -- the 4 rows must land in different groups
//    of four chunks.
// At D = 128 (256-byte rows) row bits 0-1 go to chunk bits 2-3 and row bits
// 2-3 to chunk bits 0-1. At D = 64 (128-byte rows) rows 2m and 2m + 1 already
// sit in opposite bank halves: row bit 1 goes to chunk bit 2 and row bits 2-3
// to chunk bits 0-1. (A plain row & 15 / (row >> 1) & 7 keeps the 4 rows of
// a transposing read in one group of chunks: 4- / 2-way bank conflicts.)
template <int D>
constexpr int k_swz(int row) {
  return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3))
                  : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}
// 64-byte segment swizzle of the V layout.
template <int D>
constexpr int v_swz(int row) {
  return D == 128 ? (row & 3) : ((row >> 1) & 1);
}

// Per-lane bit word of a partially visible block's kept keys, for masks with
// a window: bit p (0..31) stands for offset base + p of the lane's key (or
// row) numbering, and the kept offsets are [lo, hi] plus those <= skh (the
// sinks; empty for skh < base). Clamped bounds make any part empty.
constexpr uint32_t ones_below(int n) {   // n in [0, 32]
  return (uint32_t)(0xffffffffull >> (32 - n));
}
constexpr int clamp32(int x) { return cmin(cmax(x, 0), 32); }
constexpr uint32_t keep_word(int lo, int hi, int skh, int base) {
  return (ones_below(clamp32(hi - base + 1)) & ~ones_below(clamp32(lo - base))) |
         ones_below(clamp32(skh - base + 1));
}

// Forward (and dQ): query rows [q_lo, q_lo + BR), key blocks of BC keys; the
// walk visits n_sinkb sink blocks, then key blocks kb_lo .. kb_hi. Key block
// kb is fully visible when its keys end at or before the sequence end, and
// under the causal mask at or before the first row, and with a window start
// inside the last row's window (q_lo + BR - 1 - kb BC < window). Those bound
// one run [ka, kz] of the window's blocks. (A block fully visible only because
// all its keys are sinks is left to a masked segment.) Returns the walk steps
// of that run.
constexpr StepRange full_key_steps(int q_lo, int BR, int BC, int S, int causal, int window,
                                   int n_sinkb, int kb_lo, int kb_hi) {
  int ka = kb_lo, kz = cmin(kb_hi, S / BC - 1);
  if (causal) {
    kz = cmin(kz, (q_lo + 1) / BC - 1);
    if (window > 0) ka = cmax(ka, ceil_div(q_lo + BR - window, BC));
  }
  if (ka > kz) return StepRange{n_sinkb, n_sinkb};
  return StepRange{n_sinkb + ka - kb_lo, n_sinkb + kz - kb_lo + 1};
}

// dK/dV: keys [k_lo, k_lo + BK), query blocks of BQ rows qfirst .. qlast. Query
// block qb is fully visible when (causal) its first row is at or after the
// last key and (window) its last row is within the window of the first key,
// or every key is a sink. Returns the run as query-block offsets from qfirst.
constexpr StepRange full_query_steps(int k_lo, int BK, int BQ, int causal, int window, int n_sink,
                                     int qfirst, int qlast) {
  int qa = qfirst, qz = qlast;
  if (causal) {
    qa = cmax(qa, ceil_div(k_lo + BK - 1, BQ));
    if (window > 0 && k_lo + BK > n_sink) qz = cmin(qz, floor_div(k_lo + window - BQ, BQ));
  }
  if (qa > qz) return StepRange{0, 0};
  return StepRange{qa - qfirst, qz - qfirst + 1};
}

// The steps of F as positions in a walk over steps [it_b, it_b + n), taken in
// reverse order when rev (position t visits step it_b + n - 1 - t).
constexpr StepRange local_steps(StepRange F, int it_b, int n, bool rev) {
  int lo = rev ? it_b + n - F.hi : F.lo - it_b;
  int hi = rev ? it_b + n - F.lo : F.hi - it_b;
  lo = cmin(cmax(lo, 0), n);
  hi = cmin(cmax(hi, lo), n);
  return StepRange{lo, hi};
}

// ---- Work-group order of the forward kernels (constexpr: kernels and host) ----
//
// Work-group id -> (query block qb, batch*head bh) over a grid of nqb * BH
// work-groups. The dispatcher deals consecutive ids round-robin over the 8
// XCDs, so with BH a multiple of 8, id & 7 names the XCD; each XCD takes the
// contiguous run of BH / 8 heads [xcd * BH / 8, (xcd + 1) * BH / 8), which
// keeps query heads that share a key/value head (consecutive heads) on one
// L2.
//  * Uniform work (no mask, or a sliding window): head-major, each head's
//    query blocks in order, so the work-groups resident on an XCD cover one or
//    two heads whose keys and values fit its L2.
//  * Causal mask: the XCD's heads in groups of kOrderGroupHeads; each group
//    runs rank-major, the heaviest query block of every head of the group
//    first (balancing the causal triangle), and the next group follows. The
//    work-groups resident on an XCD then stream the keys of at most four
//    heads instead of all of the XCD's heads: on causal B4 H16 S4096 D128 the
//    L2 fetches fall from 863 to 394 MB per launch. Same-process A/B against
//    one group of all the XCD's heads: +1.4 % on that shape, +5 % at B4 H32
//    S4096, +6 % at B16 H16 S1024, +2 % at B2 H32 S8192, within noise with
//    grouped heads and at B8 H16 S2048. Groups of one or two heads lost 3-9 %
//    to the longer tail of each group.
//  * BH not a multiple of 8: rank-major over all heads.
constexpr int kOrderGroupHeads = 4;
struct Tile {
  int qb, bh;
};
constexpr Tile wg_tile(int id, int BH, int nqb, bool causal, bool window) {
  if ((BH & 7) == 0) {
    const int HX = BH >> 3;   // heads per XCD
    const int xcd = id & 7;
    const int kk = id >> 3;   // position in the XCD's sequence
    if (!causal || window) return Tile{kk % nqb, xcd * HX + kk / nqb};
    const int HG = cmin(HX, kOrderGroupHeads);
    const int g = kk / (HG * nqb);
    const int r = kk - g * HG * nqb;
    const int hn = cmin(HG, HX - g * HG);   // heads in this group
    const int rank = r / hn;
    return Tile{nqb - 1 - rank, xcd * HX + g * HG + (r - rank * hn)};
  }
  const int rank = id / BH;
  return Tile{causal ? nqb - 1 - rank : rank, id % BH};
}

inline bool fast_supported(int64_t D, int dtype) {
  return (dtype == kDtypeBF16 || dtype == kDtypeF16) && (D == 64 || D == 128);
}
inline bool bwd_supported(int64_t D, int dtype) { return fast_supported(D, dtype); }

// Arguments of one forward launch, already validated and normalised on the
// host: window >= S is folded to 0 (no window), n_sink is clamped to S, and a
// negative scale is folded into the sign of Q (neg = 1) so that c > 0.
// Query head bh (= b * H + h) reads key/value head bh / G.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  unsigned long long* block_pairs;  // optional instrumentation counter (may be null)
  const float* alibi;  // per-query-head ALiBi slopes [H], or null (no bias)
  float* o_part;       // key-split partial outputs [n_split][BH][S][D] fp32, or null
  float* lse_part;     // key-split partial LSE [n_split][BH][S] (with o_part)
  int n_split;         // key-block ranges per query block (1: no split)
  int S;        // sequence length
  int BH;       // batch * query heads
  int H;        // query heads
  int G;        // query heads per key/value head
  int nqb;      // query blocks per head = ceil(S / block_q of the chosen kernel)
  int causal;   // 0 / 1
  int window;   // 0 = none
  int n_sink;   // leading always-visible keys (only with window > 0)
  float c;      // |scale| * log2(e), at least FLT_MIN
  int neg;      // scale < 0
  int reverse;  // 1: work-groups take their tiles in reverse dispatch order (testing aid)
  int parts;    // 2 or 4: the small-grid schedule with that many key parts (8 waves); 0: off
};

// Arguments of one backward launch (validated on the host). c = scale * log2(e)
// keeps the sign of scale here: the backward kernels use the logits directly.
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;    // forward logsumexp [BH][S]
  void* dq;
  void* dk;
  void* dv;
  float* delta;        // workspace: rowsum(dO * O) [BH][Sp], 0 past S
  float* lse2;         // workspace: lse * log2(e) [BH][Sp], +inf past S
  const float* alibi;  // per-query-head slopes [H], or null
  int S, BH, H, G;     // G = query heads per key/value head
  int Sp;              // rows per head of the workspace arrays (S rounded up to the dq block)
  int nqb, nkb;        // query blocks of the dq kernel, key blocks of the dkv kernel
  int causal, window, n_sink;
  float c, scale;
  int dkv_pair;        // 1: dK/dV by two 4-wave work-groups per CU (see bwd_dkv_pair)
};

// The dK/dV kernel of a backward: two 4-wave work-groups per CU (K in
// registers, V in LDS, 32-row query tiles) when the grid fills the chip
// well, else one work-group per CU with K and V in registers. Measured on
// gfx950: the pair wins by 2-23 % on grids of 1024 work-groups and more
// (ALiBi and windows included), and by 5-8 % on 512-work-group grids whose
// key blocks see equal work (no causal mask, or a window); it loses on a
// single causal round of 512 work-groups (the first key blocks see every
// query block) and on smaller grids.
// FLASH_ATTN_DKV=1|2 forces one (tuning, tests).
bool bwd_dkv_pair(int64_t grid, bool causal, bool window);

// Which kernel and tile a problem runs with (a pure function of the shape and
// of the FLASH_ATTN_WAVES tuning override).
struct Plan {
  bool fast;
  int nw;        // waves per work-group of the fast kernel
  int block_q;   // query rows per work-group
  int block_k;   // keys per streamed block
  int parts;     // key parts of the small-grid schedule (2 or 4), or 0
};
// plain: no ALiBi and no key split (the small-grid schedule needs both).
Plan plan_fwd(int64_t BH, int64_t S, int64_t D, int dtype, bool plain, int64_t window);

}  // namespace fa
