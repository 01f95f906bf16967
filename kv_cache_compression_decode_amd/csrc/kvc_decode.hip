// Fused decode: range decode -> dequantize / anchor+delta reconstruction ->
// store into the [layer][K/V][token][channel] binary16 KV cache.
//
// CacheGen page, 核心方法: each chunk's bitstream is decoded on the GPU back
// to tensors; tokens of a 10-token group depend only on their anchor (no
// delta chain); symbols were arithmetic-coded against per channel-layer
// models, anchors and deltas separately.
//
// Work decomposition (gfx950, wave64):
//  * a workgroup owns one (layer*2+kv row, block of 64 channels) and a group
//    of chunks (normally every chunk of the call), and stages the 64
//    channels' anchor models and their delta models of every level the group
//    uses into LDS once;
//  * its W waves take the group's chunks one at a time: every lane decodes
//    the stream of its channel in the wave's chunk, and one LDS copy of the
//    models serves every chunk of the group.  One stream per wave rather
//    than several per lane in lockstep: a wave waiting for an LDS read then
//    holds up only its own stream, and the SIMDs switch between the
//    workgroups' waves (about 22 per CU for an 11-chunk call);
//  * all lanes of a wave are at the same token, so the anchor/delta switch
//    and the search depth are wave-uniform, and the 64 results of a token are
//    64 consecutive channels: one coalesced 128-byte store per stream,
//    addressed from a wave-uniform base;
//  * a symbol is the largest k with r * cum[k] <= code, found by binary
//    search with one 24-bit multiply per probe (no division): 8 steps for
//    anchors, b steps for a b-bit delta alphabet.  The entries probed by the
//    first two steps are the same for every token of a stream and sit in
//    registers, so a symbol waits on b - 1 rounds of LDS reads (the other
//    steps and its interval), not b + 1: the decoder is bound by this chain
//    of LDS latencies as much as by instruction issue;
//  * the models are staged row-interleaved (entry i of lane l in row i, a
//    128-byte row per entry index), so a probe is a constant offset from the
//    lane's current row and the symbol index is a shift of the address;
//    within a row lanes 0..31 take the low halves of the 32 dwords and lanes
//    32..63 the high halves, so a half-wave never collides on an LDS bank;
//  * stream bytes are staged per lane in a 16-byte LDS ring (stored
//    byte-reversed, so the next four bytes are one funnel shift of two
//    aligned dwords; ring dword k of a wave's lane l is the wave's LDS dword
//    64 k + l, so whatever ring positions the lanes are at, the 64 lanes of
//    a read touch 64 different banks) fed in 8-byte blocks: a lane stores the block it loaded
//    earlier only when its ring runs low (at most 8 bytes left at a group's
//    anchor, fewer than 2 before any other token) and then asks for its next
//    one, so a load has about a group of tokens to arrive;
//  * the container holds each unit's blocks in exactly that order of
//    requests (lanes in order within a step), so the wave keeps one
//    wave-uniform count of the unit's blocks handed out, a lane's block is
//    that count plus the requesting lanes below it, and a wave's loads walk
//    its unit's payload front to back: each payload byte is fetched from HBM
//    about once.  Loads go through a buffer resource bounded by the
//    container size, so a load for a lane that has no block left is
//    harmless (past the container end it reads as zero);
//  * blocks are numbered so that the groups of one (row, channel block) run
//    on the same XCD.
//
// The same file holds k_decode_refined (CacheGen page, 局限与 Future Work:
// refinement bits sent after a low-quality KV): the same decomposition, each
// lane decoding its stream's base layer and refinement layer side by side
// (two rings, one fused step per token whose two binary searches issue their
// LDS probes in lockstep) and storing binary16(fma(q, D, xh)) once.
#include "kvc_internal.h"

namespace kvc {

namespace {

constexpr uint32_t kMaxWaves = kDecodeMaxWaves;  // waves per workgroup (host picks W <= this)
constexpr uint32_t kARows = 258;    // staged anchor model rows: cum[0..256] + pad
constexpr uint32_t kDRows = 66;     // staged delta model rows: cum[0..63] + 2 pads
// staged refinement model rows for E bits: cum[0..2^E] and one pad, even
__host__ __device__ constexpr uint32_t refine_rows(uint32_t ebits) { return (1u << ebits) + 2u; }
constexpr uint32_t kRowBytes = 2 * kWave;  // one u16 entry for each of the 64 lanes
constexpr uint32_t kRing = 7;       // dwords per lane ring: 2 spare, 16 bytes, mirror of bytes 0..3
constexpr uint32_t kRingLead = 2;   // spare dwords before the ring's byte 0
constexpr uint32_t kRingStride = 4 * kWave;  // LDS bytes from a lane's ring dword k to k + 1
constexpr uint32_t kXcds = 8;

// Explicit address spaces for the LDS tables / rings and the output, so that
// every access compiles to a ds_* or global_* instruction (a generic "flat"
// access counts against both wait counters).
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) const uint8_t lds_cu8;
typedef __attribute__((address_space(1))) uint8_t gbyte;

// Position of the highest set bit counted from the top (v_ffbh_u32): 0..31,
// and all ones for 0, which only a corrupt stream can produce.
__device__ inline uint32_t ffbh(uint32_t v) {
  uint32_t r;
  __asm__("v_ffbh_u32 %0, %1" : "=v"(r) : "v"(v));
  return r;
}

// A lane's u16 column in a row of a staged model table: lanes 0..31 take
// the low halves of the row's first 32 dwords, lanes 32..63 the high halves.
__device__ inline uint32_t lane_col(uint32_t lane) { return 2 * (lane & 31) + (lane >> 5); }

// Bits 5..6 of a ring position: the first of the two ring dwords to read.
// (As a plain shift-and-mask the compiler spends one more instruction.)
__device__ inline uint32_t dword_of(uint32_t nrpos) {
  uint32_t r;
  __asm__("v_bfe_u32 %0, %1, 5, 2" : "=v"(r) : "v"(nrpos));
  return r;
}

// LDS byte address of a lane's entry `row` of a row-interleaved table.
__device__ inline uint32_t lds_addr(const lds_u32 *table) {
  return (uint32_t)(uintptr_t)table;
}
__device__ inline uint32_t lds_read_u16(uint32_t addr) {
  return *(const lds_u16 *)(uintptr_t)addr;
}

// A stream slot's container (all wave-uniform): its bounds-checked buffer
// resource, the byte offset of this unit's payload in it, and how many of the
// unit's payload blocks the wave has asked for so far.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct Source {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t ubase;
  uint32_t cnt;
};

// A lane's ring holds the stream's bytes in reverse: stream byte p sits at
// ring byte 19 - p mod 16, and ring bytes 0..3 mirror bytes 16..19.  The four
// bytes from p on are then the little-endian dword at ring byte -p mod 16,
// most significant first, and that dword lies inside the two aligned dwords
// at (-p mod 16) & 12: one paired LDS read and one funnel shift whose shift
// count is the bit position itself.  Two spare dwords precede the ring, so
// that both halves are written by the same three stores (below).  A lane's
// ring dwords are kRingStride bytes apart (the wave's 64 rings interleaved
// dword by dword).
struct Stream {
  lds_u32 *ring;        // this lane's ring dword 0 in LDS
  uint32_t code, range;
  uint32_t nrpos;       // -(bits consumed) mod 2^32 (a multiple of 8)
  uint32_t nwlim;       // -(bits written to the ring, less 16): past it fewer
                        // than 2 bytes are buffered
  u32x2 held;           // the stream's next 8-byte block, loaded ahead (one
                        // aligned register pair, the load's own destination)
  uint32_t rem;         // the stream's blocks the lane has not asked for
  uint32_t hoff;        // byte offset of the held block in the container
  uint32_t wbase;       // LDS address the next block is written from: ring
                        // dword 0, or two ring dwords before it (alternating)
  uint32_t wsum;        // the sum of those two addresses
  int32_t M;
  uint32_t dbase;       // LDS byte address of this lane's delta row 0
  uint32_t dbaseM;      // dbase + M rows: (addr - dbaseM) >> 7 is q = s - M
  uint32_t dmid;        // dbase + 2^(b-1) rows: the search's first step taken
  uint32_t d1, d2lo, d2hi;  // delta cum[2^(b-1)], cum[2^(b-2)], cum[3 2^(b-2)]
  float lo, sa7, dl7, ahat;  // sa7 = sa / 128, dl7 = dl / 128 (exact)

  // The held block, byte-reversed, into the free half of the ring: its
  // first stream byte is a multiple of 16 (dwords 4, 3 and the mirror 0) or
  // 8 past one (dwords 2, 1).  Written from w = ring dword 0 or two ring
  // dwords before it, the same three stores do both: ring dwords w+0 and w+4
  // take the block's first four bytes (the mirror and dword 4, or a spare
  // dword and dword 2), dword w+3 the other four (dword 3, or dword 1).
  __device__ inline void put_block() {
    lds_u32 *w = (lds_u32 *)(uintptr_t)wbase;
    const uint32_t lo = __builtin_bswap32(held[0]);
    w[0] = lo;
    w[4 * kWave] = lo;
    w[3 * kWave] = __builtin_bswap32(held[1]);
    wbase = wsum - wbase;
    nwlim -= 64;
  }
};

// The reading rule that fixes the payload's block order: the lanes with
// `need` store their held block into the ring and ask for their next block,
// if the stream has one; the unit's requests take consecutive payload blocks
// in lane order.  Only rings that run low do this, as late as possible, so a
// block has about a group of tokens to arrive before it is stored.
//
// Once any lane of the wave needs a block, every lane loads one: a lane that
// stores its block takes the next (a lane whose stream has none left loads
// some other block, or zeros past the container end, and never uses it), the
// others load their held block again.  No lane keeps its old register value
// across the branch, so nothing has to wait for the load before the block is
// stored, a group later.
template <class St>
__device__ inline void advance(St &s, Source &src, bool need) {
  const uint64_t need_mask = __builtin_amdgcn_ballot_w64(need);
  if (need_mask == 0) return;
  // the requesting lanes: those that need and still have a block to ask for
  const uint64_t mask = need_mask & __builtin_amdgcn_ballot_w64(s.rem != 0);
  if (need) s.put_block();
  // the unit's blocks handed out so far plus the requesting lanes below this one
  const uint32_t blk = __builtin_amdgcn_mbcnt_hi(
      (uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, src.cnt));
  s.hoff = need ? src.ubase + blk * kBlock : s.hoff;
  s.held = __builtin_amdgcn_raw_buffer_load_b64(src.rsrc, s.hoff, 0, 0);
  // one block fewer to ask for (none below zero: a lane without one did not ask)
  s.rem = need ? __builtin_elementwise_sub_sat(s.rem, 1u) : s.rem;
  src.cnt += (uint32_t)__builtin_popcountll(mask);
}
// At a group's anchor: a ring with at most 8 bytes left takes its block.
template <class St>
__device__ inline void refill(St &s, Source &src) {
  advance(s, src, (int32_t)(s.nrpos - s.nwlim) <= 48);
}
// Before every other token: a ring with fewer than 2 bytes left takes its
// block (rare).
template <class St>
__device__ inline void ensure(St &s, Source &src) { advance(s, src, s.nrpos < s.nwlim); }

// Keeps the instruction scheduler from moving code across this point: each
// binary-search probe is read, then compared, with nothing hoisted between.
#define SEARCH_BARRIER() __builtin_amdgcn_sched_barrier(0)

// The anchor model's entries at the top two levels of its search, the same
// for every token of the workgroup.
struct AnchorTop {
  uint32_t base, mid;   // LDS byte addresses of the lane's rows 0 and 128
  uint32_t c1, c2lo, c2hi;  // cum[128], cum[64], cum[192]
};

// One token of a lane's stream: range decode, dequantize.  The symbol is the
// largest k with r * cum[k] <= code (the division-free form of
// cum[k] <= floor(code / r)); kSteps binary-search steps cover indices
// [0, 2^kSteps), and delta entries past an alphabet are staged as 2^15 so
// that no product can wrap and a valid code never selects them.  Returns the
// value to store (binary16 bits, or the symbol).
template <bool kSymbols, bool kAnchor, uint32_t kSteps>
__device__ inline uint32_t step(Stream &x, const AnchorTop &at, uint64_t &lost_anchor) {
  // the next four stream bytes, most significant first
  const lds_u32 *rd =
      (const lds_u32 *)(uintptr_t)(lds_addr(x.ring) + dword_of(x.nrpos) * kRingStride);
  const uint32_t in = __builtin_amdgcn_alignbit(rd[kWave], rd[0], x.nrpos);
  const uint32_t r = x.range >> kPrec;
  // binary search; the entries of its first two steps are fixed for the
  // whole stream and held in registers, the rest are read from LDS
  constexpr uint32_t kTop = 1u << (kSteps - 1);
  const bool upper = __umul24(r, kAnchor ? at.c1 : x.d1) <= x.code;
  uint32_t a = upper ? (kAnchor ? at.mid : x.dmid) : (kAnchor ? at.base : x.dbase);
  const uint32_t p2 = upper ? (kAnchor ? at.c2hi : x.d2hi) : (kAnchor ? at.c2lo : x.d2lo);
  if (__umul24(r, p2) <= x.code) a += (kTop / 2) * kRowBytes;
  SEARCH_BARRIER();
#pragma unroll
  for (uint32_t sz = kTop / 4; sz; sz >>= 1) {
    const uint32_t probe = lds_read_u16(a + sz * kRowBytes);
    SEARCH_BARRIER();
    if (__umul24(r, probe) <= x.code) a += sz * kRowBytes;
    SEARCH_BARRIER();
  }
  const uint32_t cs = lds_read_u16(a);
  const uint32_t cn = lds_read_u16(a + kRowBytes);
  SEARCH_BARRIER();
  int32_t xq;  // 128 (symbol - M) for deltas, 128 symbol for anchors
  if constexpr (kAnchor) {
    xq = (int32_t)(a - at.base);
  } else {
    xq = (int32_t)(a - x.dbaseM);
  }
  // 24-bit multiplies: r < 2^17 and staged cumulative counts <= 2^15
  x.code -= __umul24(r, cs);
  const uint32_t range = __umul24(r, cn - cs);
  // A code at or past r * 2^15 has no symbol.  For a delta the search then
  // ends on a staged pad (2^15, as is cum[A]), so the interval is empty and
  // the range becomes 0; a zero range stays zero (r = 0 from then on) and is
  // reported at the end of the stream.  An anchor's search cannot pass symbol
  // 255, and then leaves code - r cum[255] >= r f[255], the new range, which a
  // valid code never does (code < r cum[s + 1]): the wave keeps a mask of the
  // lanes where that happened, reported at the end of the stream.
  if constexpr (kAnchor) lost_anchor |= __builtin_amdgcn_ballot_w64(x.code >= range);
  // whole bytes to shift in: 0, 1 or 2 (range >= 2^9 for a valid stream)
  const uint32_t sh = ffbh(range) & 24u;
  x.range = range << sh;
  // code << sh with the next sh / 8 stream bytes below it: one 64-bit shift
  x.code = (uint32_t)((((uint64_t)x.code << 32) | in) << sh >> 32);
  x.nrpos -= sh;
  if constexpr (kSymbols) {
    return kAnchor ? (uint32_t)xq >> 7 : (uint32_t)((xq >> 7) + x.M);
  } else {
    // 128 q is exact in binary32 and (128 q)(dl / 128) = q dl exactly, so
    // this is the single rounding of fma(q, dl, ahat)
    if constexpr (kAnchor) {
      x.ahat = __builtin_fmaf((float)xq, x.sa7, x.lo);
      // the register barrier that keeps the fma and the binary16 conversion
      // apart (see f2h) is put on ahat itself, which stays live, so the
      // conversion needs no copy of it
      __asm__("" : "+v"(x.ahat));
      return __builtin_bit_cast(uint16_t, (_Float16)x.ahat);
    } else {
      return f2h(__builtin_fmaf((float)xq, x.dl7, x.ahat));
    }
  }
}

// Stores a lane's value at its byte offset `loff` from the wave-uniform row
// base.  The empty asm makes the offset opaque at every store, so that the
// address stays "scalar base + 32-bit lane offset" (one global store with a
// scalar base, no 64-bit address arithmetic per token).
template <bool kSymbols>
__device__ inline void put(gbyte *base, uint32_t &loff, uint32_t v) {
  if constexpr (kSymbols) {
    base[loff] = (uint8_t)v;
  } else {
    __asm__("" : "+v"(loff));
    // streaming store: the kernel never reads its output back, so the rows
    // should not displace the stream blocks the lanes are still reading
    __builtin_nontemporal_store((uint16_t)v,
                                (__attribute__((address_space(1))) uint16_t *)(base + loff));
  }
}

// Wave-uniform 64-bit pointer (kept in scalar registers).
__device__ inline gbyte *uniform_ptr(gbyte *p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (gbyte *)(((uint64_t)hi << 32) | lo);
}

// The `count` delta tokens of one group.
template <bool kSymbols, uint32_t kSteps>
__device__ inline void delta_run(Stream &s, const AnchorTop &at, Source &src, gbyte *&ob, uint64_t ld,
                                 uint32_t &loff, uint32_t count, uint64_t &lost_anchor) {
  // The anchor's refill leaves at least 8 bytes in every ring and a token
  // takes at most 2 (range >= 2^24 after renormalization, a symbol's
  // frequency >= 1), so the group's first three deltas cannot run low.  A
  // corrupt stream whose range reached 0 takes 3 bytes a token, but stays
  // at 0 and is reported at the end.
  const uint32_t safe = count < 3 ? count : 3;
  uint32_t i = 0;
  for (; i < safe; ++i) {
    put<kSymbols>(ob, loff, step<kSymbols, false, kSteps>(s, at, lost_anchor));
    ob += ld;
  }
  for (; i < count; ++i) {
    ensure(s, src);
    put<kSymbols>(ob, loff, step<kSymbols, false, kSteps>(s, at, lost_anchor));
    ob += ld;
  }
}

// Every token of a lane's stream, in groups of an anchor and up to G - 1
// deltas.  The search depth of the deltas is fixed for the whole stream (the
// chunk's delta bits in this layer third), so the group loop is instantiated
// per depth and chosen once per stream.
template <bool kSymbols, uint32_t kSteps>
__device__ inline void stream_run(Stream &s, const AnchorTop &at, Source &src, gbyte *ob, uint64_t ld,
                                  uint32_t &loff, uint32_t n, uint32_t G, uint64_t &lost_anchor) {
  for (uint32_t j = 0; j < n;) {
    // after a refill at least 8 bytes are buffered: no check for the anchor
    refill(s, src);
    put<kSymbols>(ob, loff, step<kSymbols, true, 8>(s, at, lost_anchor));
    ob += ld;
    const uint32_t jend = j + G < n ? j + G : n;
    delta_run<kSymbols, kSteps>(s, at, src, ob, ld, loff, jend - j - 1, lost_anchor);
    j = jend;
  }
}

template <bool kSymbols>
__device__ inline void stream_dispatch(uint32_t steps, Stream &s, const AnchorTop &at, Source &src,
                                       gbyte *ob, uint64_t ld, uint32_t &loff, uint32_t n, uint32_t G,
                                       uint64_t &lost_anchor) {
  switch (steps) {
    case 2: stream_run<kSymbols, 2>(s, at, src, ob, ld, loff, n, G, lost_anchor); break;
    case 3: stream_run<kSymbols, 3>(s, at, src, ob, ld, loff, n, G, lost_anchor); break;
    case 4: stream_run<kSymbols, 4>(s, at, src, ob, ld, loff, n, G, lost_anchor); break;
    case 5: stream_run<kSymbols, 5>(s, at, src, ob, ld, loff, n, G, lost_anchor); break;
    default: stream_run<kSymbols, 6>(s, at, src, ob, ld, loff, n, G, lost_anchor); break;
  }
}

// ------------------------------------------------------------ refinement
// A lane's refinement stream (the second layer of its chunk): the same byte
// ring and block source as a base stream, and its two models (anchor tokens,
// other tokens), both E-bit alphabets staged like the delta models.
struct RStream {
  lds_u32 *ring;
  uint32_t code, range;
  uint32_t nrpos, nwlim;
  u32x2 held;
  uint32_t rem, hoff, wbase, wsum;
  uint32_t tab[2];   // LDS byte address of this lane's row 0: anchor tokens, other tokens
  uint32_t mid[2];   // tab + 2^(E-1) rows: the search's first step taken
  uint32_t tabM[2];  // tab + Me rows: (addr - tabM) is 128 q
  uint32_t c1[2], c2lo[2], c2hi[2];  // cum[2^(E-1)], cum[2^(E-2)], cum[3 2^(E-2)]
  float D7[2];       // Da / 128, Dd / 128 (exact: D is 0 or above 2^-100)

  // as Stream::put_block: the held block, byte-reversed, into the free half
  __device__ inline void put_block() {
    lds_u32 *w = (lds_u32 *)(uintptr_t)wbase;
    const uint32_t lo = __builtin_bswap32(held[0]);
    w[0] = lo;
    w[4 * kWave] = lo;
    w[3 * kWave] = __builtin_bswap32(held[1]);
    wbase = wsum - wbase;
    nwlim -= 64;
  }
};

// Range-decoder state update once a search has ended on the interval
// [cs, cn): the Stream::step arithmetic.  Returns whether the code is past
// the interval (code - r cs >= r (cn - cs)), which only a lost anchor shows.
template <class St>
__device__ inline bool rc_consume(St &x, uint32_t r, uint32_t cs, uint32_t cn, uint32_t in) {
  x.code -= __umul24(r, cs);
  const uint32_t range = __umul24(r, cn - cs);
  const bool past = x.code >= range;
  const uint32_t sh = ffbh(range) & 24u;
  x.range = range << sh;
  x.code = (uint32_t)((((uint64_t)x.code << 32) | in) << sh >> 32);
  x.nrpos -= sh;
  return past;
}

// One token of a lane's base and refinement streams together: both symbols
// (the base search over kSteps levels, the refinement search over E levels,
// their LDS probes issued side by side so that the two dependent chains
// overlap), then the base value xh in binary32 and binary16(fma(q, D, xh)).
template <bool kAnchor, uint32_t kSteps, uint32_t kE>
__device__ inline uint32_t rstep(Stream &x, RStream &e, const AnchorTop &at,
                                 uint64_t &lost_anchor) {
  constexpr uint32_t kind = kAnchor ? 0 : 1;
  const lds_u32 *rd =
      (const lds_u32 *)(uintptr_t)(lds_addr(x.ring) + dword_of(x.nrpos) * kRingStride);
  const uint32_t in = __builtin_amdgcn_alignbit(rd[kWave], rd[0], x.nrpos);
  const lds_u32 *erd =
      (const lds_u32 *)(uintptr_t)(lds_addr(e.ring) + dword_of(e.nrpos) * kRingStride);
  const uint32_t ein = __builtin_amdgcn_alignbit(erd[kWave], erd[0], e.nrpos);
  const uint32_t r = x.range >> kPrec;
  const uint32_t er = e.range >> kPrec;
  // the first two levels of both searches from registers
  constexpr uint32_t kTop = 1u << (kSteps - 1);
  constexpr uint32_t kETop = 1u << (kE - 1);
  const bool upper = __umul24(r, kAnchor ? at.c1 : x.d1) <= x.code;
  uint32_t a = upper ? (kAnchor ? at.mid : x.dmid) : (kAnchor ? at.base : x.dbase);
  const uint32_t p2 = upper ? (kAnchor ? at.c2hi : x.d2hi) : (kAnchor ? at.c2lo : x.d2lo);
  if (__umul24(r, p2) <= x.code) a += (kTop / 2) * kRowBytes;
  const bool eupper = __umul24(er, e.c1[kind]) <= e.code;
  uint32_t ea = eupper ? e.mid[kind] : e.tab[kind];
  const uint32_t ep2 = eupper ? e.c2hi[kind] : e.c2lo[kind];
  if (__umul24(er, ep2) <= e.code) ea += (kETop / 2) * kRowBytes;
  SEARCH_BARRIER();
  // the LDS levels, in lockstep while both searches have one
  constexpr uint32_t kLv = kSteps - 2, kELv = kE - 2;
  constexpr uint32_t kMaxLv = kLv > kELv ? kLv : kELv;
#pragma unroll
  for (uint32_t i = 0; i < kMaxLv; ++i) {
    const uint32_t sz = (kTop / 4) >> i, esz = (kETop / 4) >> i;
    uint32_t probe = 0, eprobe = 0;
    if (i < kLv) probe = lds_read_u16(a + sz * kRowBytes);
    if (i < kELv) eprobe = lds_read_u16(ea + esz * kRowBytes);
    SEARCH_BARRIER();
    if (i < kLv && __umul24(r, probe) <= x.code) a += sz * kRowBytes;
    if (i < kELv && __umul24(er, eprobe) <= e.code) ea += esz * kRowBytes;
    SEARCH_BARRIER();
  }
  const uint32_t cs = lds_read_u16(a);
  const uint32_t cn = lds_read_u16(a + kRowBytes);
  const uint32_t ecs = lds_read_u16(ea);
  const uint32_t ecn = lds_read_u16(ea + kRowBytes);
  SEARCH_BARRIER();
  // base: as Stream::step (a lost anchor is recorded the same way)
  const int32_t xq = kAnchor ? (int32_t)(a - at.base) : (int32_t)(a - x.dbaseM);
  const bool past = rc_consume(x, r, cs, cn, in);
  if constexpr (kAnchor) lost_anchor |= __builtin_amdgcn_ballot_w64(past);
  const int32_t eq = (int32_t)(ea - e.tabM[kind]);
  rc_consume(e, er, ecs, ecn, ein);
  float xh;
  if constexpr (kAnchor) {
    x.ahat = __builtin_fmaf((float)xq, x.sa7, x.lo);
    xh = x.ahat;
  } else {
    xh = __builtin_fmaf((float)xq, x.dl7, x.ahat);
  }
  return f2h(__builtin_fmaf((float)eq, e.D7[kind], xh));
}

// Every token of a lane's base and refinement streams, group by group; the
// two streams follow the same reading rule, each over its own container.
template <uint32_t kSteps, uint32_t kE>
__device__ inline void refined_run(Stream &s, RStream &e, const AnchorTop &at, Source &src,
                                   Source &rsrc, gbyte *ob, uint64_t ld, uint32_t &loff,
                                   uint32_t n, uint32_t G, uint64_t &lost_anchor) {
  for (uint32_t j = 0; j < n;) {
    refill(s, src);
    refill(e, rsrc);
    put<false>(ob, loff, rstep<true, 8, kE>(s, e, at, lost_anchor));
    ob += ld;
    const uint32_t jend = j + G < n ? j + G : n;
    const uint32_t count = jend - j - 1;
    for (uint32_t i = 0; i < count; ++i) {
      // the first three deltas after an anchor's refill cannot run low
      if (i >= 3) {
        ensure(s, src);
        ensure(e, rsrc);
      }
      put<false>(ob, loff, rstep<false, kSteps, kE>(s, e, at, lost_anchor));
      ob += ld;
    }
    j = jend;
  }
}

template <uint32_t kE>
__device__ inline void refined_run_b(uint32_t b, Stream &s, RStream &e, const AnchorTop &at,
                                     Source &src, Source &rsrc, gbyte *ob, uint64_t ld,
                                     uint32_t &loff, uint32_t n, uint32_t G,
                                     uint64_t &lost_anchor) {
  switch (b) {
    case 2: refined_run<2, kE>(s, e, at, src, rsrc, ob, ld, loff, n, G, lost_anchor); break;
    case 3: refined_run<3, kE>(s, e, at, src, rsrc, ob, ld, loff, n, G, lost_anchor); break;
    case 4: refined_run<4, kE>(s, e, at, src, rsrc, ob, ld, loff, n, G, lost_anchor); break;
    case 5: refined_run<5, kE>(s, e, at, src, rsrc, ob, ld, loff, n, G, lost_anchor); break;
    default: refined_run<6, kE>(s, e, at, src, rsrc, ob, ld, loff, n, G, lost_anchor); break;
  }
}

}  // namespace

template <bool kSymbols>
__global__ __launch_bounds__(kMaxWaves *kWave) void k_decode(
    Desc d, const ChunkInfo *__restrict__ ci, const DecodeGroup *__restrict__ groups,
    uint32_t n_groups, uint32_t n_units, const uint8_t *__restrict__ valid,
    const uint32_t *__restrict__ offsets, const uint8_t *__restrict__ tables,
    int32_t *status) {
  // ---- which (unit, chunk group) this block owns (XCD-aware numbering)
  const uint32_t id = blockIdx.x;
  const uint32_t local = id / kXcds;
  const uint32_t unit = (local / n_groups) * kXcds + id % kXcds;
  const uint32_t grp = local % n_groups;
  if (unit >= n_units) return;
  const uint32_t ncb = (d.C + kWave - 1) / kWave;
  const uint32_t row = unit / ncb, cb = unit % ncb;
  const uint32_t c0 = cb * kWave;
  const uint32_t nv = d.C - c0 < kWave ? d.C - c0 : kWave;
  const uint32_t m0 = row * d.C + c0;
  const uint32_t S = n_streams(d);
  const DecodeGroup gp = groups[grp];
  const uint32_t level_mask = gp.level;  // bit l: the group has chunks of level l
  const uint32_t nlev_used = __builtin_popcount(level_mask);
  const uint32_t n_waves = blockDim.x / kWave;

  extern __shared__ uint32_t lds_raw[];
  lds_u32 *lds = (lds_u32 *)lds_raw;
  lds_u32 *sA = lds;                                    // [kARows][64] u16 anchor cum
  lds_u32 *sD = sA + kARows * kWave / 2;                // [levels used][kDRows][64] u16 delta cum
  lds_u32 *sR = sD + nlev_used * kDRows * kWave / 2;    // [waves][kRing][64] rings
  lds_u16 *hA = (lds_u16 *)sA;
  lds_u16 *hD = (lds_u16 *)sD;

  // ---- stage the 64 channels' anchor models and the used levels' delta
  // models, row-interleaved: entry i of lane l at u16 index
  // i * 64 + lane_col(l), so the 32 lanes of a half-wave always read 32
  // different dwords of their rows, one per bank, whatever rows they are at.
  const uint32_t tid = threadIdx.x;
  {
    const uint32_t *gA = reinterpret_cast<const uint32_t *>(tables + kTablesHdr) +
                         (uint64_t)m0 * (kAnchorStride / 2);
    for (uint32_t i = tid; i < nv * (kARows / 2); i += blockDim.x) {
      const uint32_t w = i / nv, l = i % nv;
      const uint32_t v = gA[(uint64_t)l * (kAnchorStride / 2) + w];
      hA[(2 * w) * kWave + lane_col(l)] = (uint16_t)v;
      hA[(2 * w + 1) * kWave + lane_col(l)] = (uint16_t)(v >> 16);
    }
    uint32_t slot = 0;
    for (uint32_t lv = 0; lv < d.nlev; ++lv) {
      if (!((level_mask >> lv) & 1u)) continue;
      const uint32_t *gD = reinterpret_cast<const uint32_t *>(
                               tables + kTablesHdr + (uint64_t)S * kAnchorStride * 2) +
                           ((uint64_t)lv * S + m0) * (kDeltaStride / 2);
      lds_u16 *dst = hD + slot * kDRows * kWave;
      for (uint32_t i = tid; i < nv * (kDRows / 2); i += blockDim.x) {
        const uint32_t w = i / nv, l = i % nv;
        const uint32_t v =
            w < kDeltaStride / 2 ? gD[(uint64_t)l * (kDeltaStride / 2) + w] : 0xFFFFFFFFu;
        // entries past cum[A] (0xFFFF pads) become 2^15 = cum[A]
        const uint32_t e0 = v & 0xFFFFu, e1 = v >> 16;
        dst[(2 * w) * kWave + lane_col(l)] = (uint16_t)(e0 == 0xFFFFu ? kTot : e0);
        dst[(2 * w + 1) * kWave + lane_col(l)] = (uint16_t)(e1 == 0xFFFFu ? kTot : e1);
      }
      ++slot;
    }
  }
  __syncthreads();
  const uint32_t lane = tid % kWave;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  if (lane >= nv) return;

  AnchorTop at;
  at.base = lds_addr(sA) + 2 * lane_col(lane);
  at.mid = at.base + 128 * kRowBytes;
  at.c1 = lds_read_u16(at.mid);
  at.c2lo = lds_read_u16(at.base + 64 * kRowBytes);
  at.c2hi = lds_read_u16(at.base + 192 * kRowBytes);
  const uint32_t third = third_of(row >> 1, d.L);
  const uint32_t esz = kSymbols ? 1u : 2u;
  const uint64_t ld = (uint64_t)d.C * esz;
  const uint32_t m = m0 + lane;
  // this wave's ring (one register holds its address, so that a ring read
  // is one bit-field extract and one shift-add)
  uint32_t ring_addr = lds_addr(sR + (wave * kRing + kRingLead) * kWave + lane);
  __asm__ volatile("" : "+v"(ring_addr));
  uint32_t loff = lane * esz;
  __asm__ volatile("" : "+v"(loff));

  for (uint32_t i = wave; i < gp.count; i += n_waves) {
    const uint32_t k = gp.start + i;
    if (!valid[k]) continue;
    const ChunkInfo c = ci[k];
    Stream s;
    s.ring = (lds_u32 *)(uintptr_t)ring_addr;
    const uint32_t lslot = __builtin_popcount(level_mask & ((1u << c.level) - 1u));
    s.dbase = lds_addr(sD) + lslot * kDRows * kRowBytes + 2 * lane_col(lane);
    const uint32_t b = __builtin_amdgcn_readfirstlane(d.bits[c.level][third]);
    s.M = (1 << (b - 1)) - 1;
    s.dbaseM = s.dbase + (uint32_t)s.M * kRowBytes;
    s.dmid = s.dbase + (1u << (b - 1)) * kRowBytes;
    s.d1 = lds_read_u16(s.dmid);
    s.d2lo = lds_read_u16(s.dbase + (1u << (b - 2)) * kRowBytes);
    s.d2hi = lds_read_u16(s.dbase + 3u * (1u << (b - 2)) * kRowBytes);
    const uint32_t *rec = reinterpret_cast<const uint32_t *>(c.records + (uint64_t)m * kRecBytes);
    s.lo = __builtin_bit_cast(float, rec[0]);
    // sa / 128 and dl / 128 are exact: sa is 0 or at least 2^-24 / 255 (a
    // binary16 difference), dl is 0 or above 2^-70 (a difference of a
    // binary16 value and an anchor on a 2^-55 grid), far from subnormals
    s.sa7 = __builtin_bit_cast(float, rec[1]) * 0.0078125f;
    s.dl7 = __builtin_bit_cast(float, rec[2]) * 0.0078125f;
    const uint32_t nblk = (uint32_t)(pad8(rec[3]) / kBlock);
    // containers are below 2^32 bytes (checked on the host); this unit's
    // payload starts at its first stream's block offset
    Source src;
    src.rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)c.cont, (short)0,
                                                 (int)(uint32_t)c.cont_bytes, kBufferWord3);
    src.ubase = (uint32_t)(kHdrBytes + (uint64_t)kRecBytes * S) + offsets[(uint64_t)k * S + m0];
    src.cnt = 0;
    gbyte *ob = uniform_ptr((gbyte *)c.out +
                            (((uint64_t)row * c.out_tokens + c.first_token) * d.C + c0) * esz);
    s.ahat = 0.0f;
    // start of the reading rule: every lane asks for its blocks 0, 1 and 2
    // (block outer, lane inner); 0 and 1 fill the ring, 2 is held.  A lane
    // without the block loads some other block and never uses it.
    uint32_t blk[3][2];
#pragma unroll
    for (uint32_t q = 0; q < 3; ++q) {
      const uint64_t mask = __builtin_amdgcn_ballot_w64(q < nblk);
      const uint32_t pos = src.cnt + lanes_below(mask);
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(src.rsrc, src.ubase + pos * kBlock, 0, 0);
      blk[q][0] = v[0];
      blk[q][1] = v[1];
      if (q == 2) s.hoff = src.ubase + pos * kBlock;
      src.cnt += (uint32_t)__builtin_popcountll(mask);
    }
    s.rem = nblk < 3 ? 0u : nblk - 3;
    s.ring[4 * kWave] = __builtin_bswap32(blk[0][0]);
    s.ring[3 * kWave] = __builtin_bswap32(blk[0][1]);
    s.ring[2 * kWave] = __builtin_bswap32(blk[1][0]);
    s.ring[1 * kWave] = __builtin_bswap32(blk[1][1]);
    s.ring[0] = __builtin_bswap32(blk[0][0]);
    s.held[0] = blk[2][0];
    s.held[1] = blk[2][1];
    s.nwlim = 0u - (128 - 16);
    s.wbase = ring_addr;  // block 2 goes to dwords 4, 3 and the mirror
    s.wsum = 2u * ring_addr - 2u * kRingStride;
    s.code = bswap32(blk[0][0]);
    s.nrpos = 0u - 32;
    s.range = 0xFFFFFFFFu;

    uint64_t lost_anchor = 0;
    stream_dispatch<kSymbols>(b, s, at, src, ob, ld, loff, c.n_tokens, d.G, lost_anchor);
    // a valid stream ends exactly at its last byte, with every block asked for
    const uint32_t nbytes =
        reinterpret_cast<const uint32_t *>(ci[k].records + (uint64_t)m * kRecBytes)[3];
    if (s.range == 0 || s.nrpos != 0u - 8 * nbytes || s.rem != 0 || ((lost_anchor >> lane) & 1))
      set_status(status, KVC_ERR_CORRUPT_STREAM);
  }
}

// Decode of base and refinement layers in one launch: the same work
// decomposition as k_decode; each lane decodes its base stream and its
// refinement stream token by token and stores binary16(fma(q, D, xh)).
// Groups hold chunks of one level (the host forms them so), whose base delta
// models and two refinement models are staged beside the anchor models.
__global__ __launch_bounds__(kMaxWaves *kWave) void k_decode_refined(
    Desc d, uint32_t ebits, const ChunkInfo *__restrict__ ci, const ChunkInfo *__restrict__ rci,
    const DecodeGroup *__restrict__ groups, uint32_t n_groups, uint32_t n_units,
    const uint8_t *__restrict__ valid, const uint8_t *__restrict__ rvalid,
    const uint32_t *__restrict__ offsets, const uint32_t *__restrict__ roffsets,
    const uint8_t *__restrict__ tables, const uint8_t *__restrict__ rtables, int32_t *status) {
  const uint32_t id = blockIdx.x;
  const uint32_t local = id / kXcds;
  const uint32_t unit = (local / n_groups) * kXcds + id % kXcds;
  const uint32_t grp = local % n_groups;
  if (unit >= n_units) return;
  const uint32_t ncb = (d.C + kWave - 1) / kWave;
  const uint32_t row = unit / ncb, cb = unit % ncb;
  const uint32_t c0 = cb * kWave;
  const uint32_t nv = d.C - c0 < kWave ? d.C - c0 : kWave;
  const uint32_t m0 = row * d.C + c0;
  const uint32_t S = n_streams(d);
  const DecodeGroup gp = groups[grp];
  const uint32_t level_mask = gp.level;  // bit l: the group has chunks of level l
  const uint32_t n_waves = blockDim.x / kWave;
  const uint32_t erows = refine_rows(ebits);
  const uint32_t slot_rows = kDRows + 2 * erows;
  // the refinement tables were made for this descriptor, E and these base
  // tables (their base id is the base tables' profile id)
  if (!refine_tables_match(d, ebits, rtables) ||
      *reinterpret_cast<const uint64_t *>(rtables + 56) !=
          *reinterpret_cast<const uint64_t *>(tables + 48)) {
    if (threadIdx.x == 0) set_status(status, KVC_ERR_PROFILE_MISMATCH);
    return;
  }

  extern __shared__ uint32_t lds_raw[];
  lds_u32 *lds = (lds_u32 *)lds_raw;
  // [kARows][64] anchor cum, then one slot per level the group uses: base
  // delta cum [kDRows][64], refinement cum of anchor tokens and of the other
  // tokens [erows][64] each; then the rings [waves][2][kRing][64]
  lds_u32 *sA = lds;
  lds_u32 *sL = sA + kARows * kWave / 2;
  lds_u32 *sR = sL + __builtin_popcount(level_mask) * slot_rows * kWave / 2;
  lds_u16 *hA = (lds_u16 *)sA;

  const uint32_t tid = threadIdx.x;
  {
    const uint32_t *gA = reinterpret_cast<const uint32_t *>(tables + kTablesHdr) +
                         (uint64_t)m0 * (kAnchorStride / 2);
    for (uint32_t i = tid; i < nv * (kARows / 2); i += blockDim.x) {
      const uint32_t w = i / nv, l = i % nv;
      const uint32_t v = gA[(uint64_t)l * (kAnchorStride / 2) + w];
      hA[(2 * w) * kWave + lane_col(l)] = (uint16_t)v;
      hA[(2 * w + 1) * kWave + lane_col(l)] = (uint16_t)(v >> 16);
    }
    // per level: the base deltas, the refinement of anchor tokens and of the
    // other tokens; entries past an alphabet (0xFFFF pads) become 2^15 = cum[A]
    uint32_t slot = 0;
    for (uint32_t lv = 0; lv < d.nlev; ++lv) {
      if (!((level_mask >> lv) & 1u)) continue;
      const uint32_t *src3[3] = {
          reinterpret_cast<const uint32_t *>(tables + kTablesHdr +
                                             (uint64_t)S * kAnchorStride * 2) +
              ((uint64_t)lv * S + m0) * (kDeltaStride / 2),
          reinterpret_cast<const uint32_t *>(rtables + kTablesHdr) +
              ((uint64_t)lv * S + m0) * (kDeltaStride / 2),
          reinterpret_cast<const uint32_t *>(rtables + kTablesHdr) +
              (((uint64_t)d.nlev + lv) * S + m0) * (kDeltaStride / 2)};
      lds_u16 *sbase = (lds_u16 *)(sL + slot * slot_rows * kWave / 2);
      for (uint32_t t = 0; t < 3; ++t) {
        const uint32_t rows = t == 0 ? kDRows : erows;
        lds_u16 *dst = sbase + (t == 0 ? 0u : (kDRows + (t - 1) * erows) * kWave);
        for (uint32_t i = tid; i < nv * (rows / 2); i += blockDim.x) {
          const uint32_t w = i / nv, l = i % nv;
          const uint32_t v =
              w < kDeltaStride / 2 ? src3[t][(uint64_t)l * (kDeltaStride / 2) + w] : 0xFFFFFFFFu;
          const uint32_t e0 = v & 0xFFFFu, e1 = v >> 16;
          dst[(2 * w) * kWave + lane_col(l)] = (uint16_t)(e0 == 0xFFFFu ? kTot : e0);
          dst[(2 * w + 1) * kWave + lane_col(l)] = (uint16_t)(e1 == 0xFFFFu ? kTot : e1);
        }
      }
      ++slot;
    }
  }
  __syncthreads();
  const uint32_t lane = tid % kWave;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  if (lane >= nv) return;

  AnchorTop at;
  at.base = lds_addr(sA) + 2 * lane_col(lane);
  at.mid = at.base + 128 * kRowBytes;
  at.c1 = lds_read_u16(at.mid);
  at.c2lo = lds_read_u16(at.base + 64 * kRowBytes);
  at.c2hi = lds_read_u16(at.base + 192 * kRowBytes);
  const uint32_t third = third_of(row >> 1, d.L);
  const uint64_t ld = (uint64_t)d.C * 2u;
  const uint32_t m = m0 + lane;
  const int32_t Me = (1 << (ebits - 1)) - 1;
  const uint32_t etop = 1u << (ebits - 1);
  uint32_t ring_addr = lds_addr(sR + (2 * wave * kRing + kRingLead) * kWave + lane);
  __asm__ volatile("" : "+v"(ring_addr));
  const uint32_t rring_addr = ring_addr + kRing * kRingStride;
  uint32_t loff = lane * 2u;
  __asm__ volatile("" : "+v"(loff));

  for (uint32_t i = wave; i < gp.count; i += n_waves) {
    const uint32_t k = gp.start + i;
    if (!valid[k] || !rvalid[k]) continue;
    const ChunkInfo c = ci[k];
    const ChunkInfo rc = rci[k];
    // the refinement must be of the base container's chunk (both headers
    // were checked by the index; the token each was encoded from is at 28)
    if (*reinterpret_cast<const uint32_t *>(c.cont + 28) !=
        *reinterpret_cast<const uint32_t *>(rc.cont + 28)) {
      set_status(status, KVC_ERR_CORRUPT_STREAM);
      continue;
    }
    // ---- the base stream, as in k_decode
    Stream s;
    s.ring = (lds_u32 *)(uintptr_t)ring_addr;
    const uint32_t lslot = __builtin_popcount(level_mask & ((1u << c.level) - 1u));
    const uint32_t slot_addr = lds_addr(sL) + lslot * slot_rows * kRowBytes + 2 * lane_col(lane);
    s.dbase = slot_addr;
    const uint32_t b = __builtin_amdgcn_readfirstlane(d.bits[c.level][third]);
    s.M = (1 << (b - 1)) - 1;
    s.dbaseM = s.dbase + (uint32_t)s.M * kRowBytes;
    s.dmid = s.dbase + (1u << (b - 1)) * kRowBytes;
    s.d1 = lds_read_u16(s.dmid);
    s.d2lo = lds_read_u16(s.dbase + (1u << (b - 2)) * kRowBytes);
    s.d2hi = lds_read_u16(s.dbase + 3u * (1u << (b - 2)) * kRowBytes);
    const uint32_t *rec = reinterpret_cast<const uint32_t *>(c.records + (uint64_t)m * kRecBytes);
    s.lo = __builtin_bit_cast(float, rec[0]);
    s.sa7 = __builtin_bit_cast(float, rec[1]) * 0.0078125f;
    s.dl7 = __builtin_bit_cast(float, rec[2]) * 0.0078125f;
    const uint32_t nblk = (uint32_t)(pad8(rec[3]) / kBlock);
    Source src;
    src.rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)c.cont, (short)0,
                                                 (int)(uint32_t)c.cont_bytes, kBufferWord3);
    src.ubase = (uint32_t)(kHdrBytes + (uint64_t)kRecBytes * S) + offsets[(uint64_t)k * S + m0];
    src.cnt = 0;
    s.ahat = 0.0f;
    // ---- the refinement stream
    RStream e;
    e.ring = (lds_u32 *)(uintptr_t)rring_addr;
    e.tab[0] = slot_addr + kDRows * kRowBytes;
    e.tab[1] = e.tab[0] + erows * kRowBytes;
    for (uint32_t t = 0; t < 2; ++t) {
      e.tabM[t] = e.tab[t] + (uint32_t)Me * kRowBytes;
      e.mid[t] = e.tab[t] + etop * kRowBytes;
      e.c1[t] = lds_read_u16(e.mid[t]);
      e.c2lo[t] = lds_read_u16(e.tab[t] + (etop / 2) * kRowBytes);
      e.c2hi[t] = lds_read_u16(e.tab[t] + 3u * (etop / 2) * kRowBytes);
    }
    const uint32_t *rrec = reinterpret_cast<const uint32_t *>(rc.records + (uint64_t)m * kRecBytes);
    e.D7[0] = __builtin_bit_cast(float, rrec[0]) * 0.0078125f;
    e.D7[1] = __builtin_bit_cast(float, rrec[1]) * 0.0078125f;
    const uint32_t rnblk = (uint32_t)(pad8(rrec[3]) / kBlock);
    Source rsrc;
    rsrc.rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)rc.cont, (short)0,
                                                  (int)(uint32_t)rc.cont_bytes, kBufferWord3);
    rsrc.ubase = (uint32_t)(kHdrBytes + (uint64_t)kRecBytes * S) + roffsets[(uint64_t)k * S + m0];
    rsrc.cnt = 0;
    // start of the reading rule for both: blocks 0, 1 and 2 of every lane
    // (block outer, lane inner); 0 and 1 fill the ring, 2 is held
    uint32_t blk[3][2], rblk[3][2];
#pragma unroll
    for (uint32_t q = 0; q < 3; ++q) {
      const uint64_t mask = __builtin_amdgcn_ballot_w64(q < nblk);
      const uint32_t pos = src.cnt + lanes_below(mask);
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(src.rsrc, src.ubase + pos * kBlock, 0, 0);
      blk[q][0] = v[0];
      blk[q][1] = v[1];
      if (q == 2) s.hoff = src.ubase + pos * kBlock;
      src.cnt += (uint32_t)__builtin_popcountll(mask);
      const uint64_t rmask = __builtin_amdgcn_ballot_w64(q < rnblk);
      const uint32_t rpos = rsrc.cnt + lanes_below(rmask);
      const auto rv =
          __builtin_amdgcn_raw_buffer_load_b64(rsrc.rsrc, rsrc.ubase + rpos * kBlock, 0, 0);
      rblk[q][0] = rv[0];
      rblk[q][1] = rv[1];
      if (q == 2) e.hoff = rsrc.ubase + rpos * kBlock;
      rsrc.cnt += (uint32_t)__builtin_popcountll(rmask);
    }
    s.rem = nblk < 3 ? 0u : nblk - 3;
    s.ring[4 * kWave] = __builtin_bswap32(blk[0][0]);
    s.ring[3 * kWave] = __builtin_bswap32(blk[0][1]);
    s.ring[2 * kWave] = __builtin_bswap32(blk[1][0]);
    s.ring[1 * kWave] = __builtin_bswap32(blk[1][1]);
    s.ring[0] = __builtin_bswap32(blk[0][0]);
    s.held[0] = blk[2][0];
    s.held[1] = blk[2][1];
    s.nwlim = 0u - (128 - 16);
    s.wbase = ring_addr;
    s.wsum = 2u * ring_addr - 2u * kRingStride;
    s.code = bswap32(blk[0][0]);
    s.nrpos = 0u - 32;
    s.range = 0xFFFFFFFFu;
    e.rem = rnblk < 3 ? 0u : rnblk - 3;
    e.ring[4 * kWave] = __builtin_bswap32(rblk[0][0]);
    e.ring[3 * kWave] = __builtin_bswap32(rblk[0][1]);
    e.ring[2 * kWave] = __builtin_bswap32(rblk[1][0]);
    e.ring[1 * kWave] = __builtin_bswap32(rblk[1][1]);
    e.ring[0] = __builtin_bswap32(rblk[0][0]);
    e.held[0] = rblk[2][0];
    e.held[1] = rblk[2][1];
    e.nwlim = 0u - (128 - 16);
    e.wbase = rring_addr;
    e.wsum = 2u * rring_addr - 2u * kRingStride;
    e.code = bswap32(rblk[0][0]);
    e.nrpos = 0u - 32;
    e.range = 0xFFFFFFFFu;

    gbyte *ob = uniform_ptr((gbyte *)c.out +
                            (((uint64_t)row * c.out_tokens + c.first_token) * d.C + c0) * 2u);
    uint64_t lost_anchor = 0;
    switch (ebits) {
      case 2: refined_run_b<2>(b, s, e, at, src, rsrc, ob, ld, loff, c.n_tokens, d.G, lost_anchor); break;
      case 3: refined_run_b<3>(b, s, e, at, src, rsrc, ob, ld, loff, c.n_tokens, d.G, lost_anchor); break;
      case 4: refined_run_b<4>(b, s, e, at, src, rsrc, ob, ld, loff, c.n_tokens, d.G, lost_anchor); break;
      case 5: refined_run_b<5>(b, s, e, at, src, rsrc, ob, ld, loff, c.n_tokens, d.G, lost_anchor); break;
      default: refined_run_b<6>(b, s, e, at, src, rsrc, ob, ld, loff, c.n_tokens, d.G, lost_anchor); break;
    }
    const uint32_t nbytes =
        reinterpret_cast<const uint32_t *>(ci[k].records + (uint64_t)m * kRecBytes)[3];
    const uint32_t rnbytes =
        reinterpret_cast<const uint32_t *>(rci[k].records + (uint64_t)m * kRecBytes)[3];
    if (s.range == 0 || s.nrpos != 0u - 8 * nbytes || s.rem != 0 || ((lost_anchor >> lane) & 1) ||
        e.range == 0 || e.nrpos != 0u - 8 * rnbytes || e.rem != 0)
      set_status(status, KVC_ERR_CORRUPT_STREAM);
  }
}

size_t decode_refined_lds_bytes(uint32_t levels, uint32_t ebits, uint32_t waves) {
  return (size_t)kARows * kRowBytes +
         (size_t)levels * (kDRows + 2 * refine_rows(ebits)) * kRowBytes +
         sizeof(uint32_t) * (size_t)waves * kWave * 2 * kRing;
}

hipError_t launch_decode_refined(const Desc &d, uint32_t ebits, const ChunkInfo *dev_chunks,
                                 const ChunkInfo *dev_rchunks, const DecodeGroup *groups,
                                 uint32_t n_groups, uint32_t levels, uint32_t waves, const uint8_t *valid,
                                 const uint8_t *rvalid, const uint32_t *offsets,
                                 const uint32_t *roffsets, const uint8_t *tables,
                                 const uint8_t *rtables, int32_t *status, hipStream_t stream) {
  const uint32_t ncb = (d.C + kWave - 1) / kWave;
  const uint32_t n_units = 2u * d.L * ncb;
  const uint64_t blocks = (uint64_t)((n_units + kXcds - 1) / kXcds) * kXcds * n_groups;
  hipLaunchKernelGGL(k_decode_refined, dim3((uint32_t)blocks), dim3(waves * kWave),
                     decode_refined_lds_bytes(levels, ebits, waves), stream, d, ebits, dev_chunks, dev_rchunks,
                     groups, n_groups, n_units, valid, rvalid, offsets, roffsets, tables, rtables,
                     status);
  return hipGetLastError();
}

size_t decode_lds_bytes(uint32_t levels, uint32_t waves) {
  return (size_t)kARows * kRowBytes + (size_t)levels * kDRows * kRowBytes +
         sizeof(uint32_t) * (size_t)waves * kWave * kRing;
}

hipError_t launch_decode(const Desc &d, const ChunkInfo *dev_chunks, const DecodeGroup *groups,
                         uint32_t n_groups, uint32_t levels, uint32_t waves, const uint8_t *valid,
                         const uint32_t *offsets, const uint8_t *tables, bool symbols,
                         int32_t *status, hipStream_t stream) {
  const uint32_t ncb = (d.C + kWave - 1) / kWave;
  const uint32_t n_units = 2u * d.L * ncb;
  const uint64_t blocks = (uint64_t)((n_units + kXcds - 1) / kXcds) * kXcds * n_groups;
  const size_t lds = decode_lds_bytes(levels, waves);
  if (symbols)
    hipLaunchKernelGGL(k_decode<true>, dim3((uint32_t)blocks), dim3(waves * kWave), lds, stream,
                       d, dev_chunks, groups, n_groups, n_units, valid, offsets, tables, status);
  else
    hipLaunchKernelGGL(k_decode<false>, dim3((uint32_t)blocks), dim3(waves * kWave), lds, stream,
                       d, dev_chunks, groups, n_groups, n_units, valid, offsets, tables, status);
  return hipGetLastError();
}

}  // namespace kvc
