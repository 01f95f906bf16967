// Encode: binary16 KV [L][2][T][C] -> one container per chunk.
//
// CacheGen page, 核心方法: chunks of ~1.5K tokens coded independently;
// change-based encoding (10-token groups, 8-bit anchor, deltas to the
// anchor); layer-wise delta quantization (coarser for deeper thirds);
// arithmetic coding with per channel-layer models.
//
// Kernels (a workgroup per (row, 64-channel block, group of chunks) stages
// the 64 channels' models once; its waves take the group's chunks in turn;
// lane = channel, so every token's 64 inputs are one coalesced 128-byte
// load):
//   k_encode_stats : per stream lo / sa / dl and the exact coded length
//                    (the length depends only on the range evolution, so no
//                    bytes are produced); records go to the workspace;
//   (index kernels): per-stream payload offsets from those lengths;
//   k_encode_layout: container start offsets, capacity check;
//   k_encode_emit  : quantize and range-encode into the final position; the
//                    output bytes wait in registers (6 to 11 of them) until
//                    a carry can no longer reach them, so a carry is one
//                    add-with-carry chain and no lane branches per byte; a
//                    (chunk, unit) where a carry had to pass every held byte
//                    (a run of 6 or more 0xFF bytes) or a lane's block queue
//                    ran full is listed for the next kernel;
//   k_encode_redo  : the listed (chunk, unit)s again, one stream per lane:
//                    each stream's bytes into linear scratch with the carry
//                    added into them, then the reading rule replayed for the
//                    unit to put every block in its place;
//   k_encode_header: the 64-byte headers.
#include "kvc_internal.h"

namespace kvc {

namespace {

constexpr uint32_t kXcds = 8;

// Leading zero bits of a nonzero word (v_ffbh_u32, no test for zero).
__device__ inline uint32_t lead_zeros(uint32_t v) {
  uint32_t r;
  __asm__("v_ffbh_u32 %0, %1" : "=v"(r) : "v"(v));
  return r;
}
constexpr uint32_t kEA = 133;  // dwords per staged anchor model (cum[0..256] + pad; odd)
constexpr uint32_t kED = 33;   // dwords per staged delta model (cum[0..63] + pad; odd)

// The 64 channels' anchor models and the delta models of every level in
// `level_mask`, one row per lane at odd dword strides (lanes indexing their
// own rows hit different banks more often than not).
__device__ inline void stage_tables(const Desc &d, const uint8_t *tables, uint32_t m0,
                                    uint32_t nv, uint32_t level_mask, uint32_t *sA,
                                    uint32_t *sD) {
  const uint32_t S = n_streams(d);
  const uint32_t *gA = reinterpret_cast<const uint32_t *>(tables + kTablesHdr) +
                       (uint64_t)m0 * (kAnchorStride / 2);
  for (uint32_t i = threadIdx.x; i < nv * (kAnchorStride / 2); i += blockDim.x) {
    const uint32_t l = i / (kAnchorStride / 2), w = i % (kAnchorStride / 2);
    if (w < kEA) sA[l * kEA + w] = gA[i];
  }
  uint32_t slot = 0;
  for (uint32_t lv = 0; lv < d.nlev; ++lv) {
    if (!((level_mask >> lv) & 1u)) continue;
    const uint32_t *gD = reinterpret_cast<const uint32_t *>(
                             tables + kTablesHdr + (uint64_t)S * kAnchorStride * 2) +
                         ((uint64_t)lv * S + m0) * (kDeltaStride / 2);
    uint32_t *dst = sD + slot * kWave * kED;
    for (uint32_t i = threadIdx.x; i < nv * (kDeltaStride / 2); i += blockDim.x) {
      const uint32_t l = i / (kDeltaStride / 2), w = i % (kDeltaStride / 2);
      dst[l * kED + w] = gD[i];
    }
    ++slot;
  }
}

// A staged model is well formed: cum[0] = 0, cum[A] = 2^15, and every
// symbol's frequency at least 1.
__device__ inline bool model_ok(const uint16_t *cum, uint32_t A) {
  bool ok = cum[0] == 0 && cum[A] == kTot;
  for (uint32_t s = 0; s < A; ++s) ok = ok && cum[s] < cum[s + 1];
  return ok;
}

// Which (unit, group) a block owns: the groups of one (row, channel block)
// on the same XCD.
struct EncodeBlock {
  uint32_t unit, grp;
};
__device__ inline EncodeBlock encode_block(uint32_t n_groups) {
  const uint32_t id = blockIdx.x;
  const uint32_t local = id / kXcds;
  return {(local / n_groups) * kXcds + id % kXcds, local % n_groups};
}

// Entries of the per-lane queue of payload blocks asked for (by the reading
// rule) but not yet written.  The decoder asks for a block about 3 blocks
// ahead of what it has consumed, and the encoder holds back at most 11
// bytes, so about 5 entries are ever in use; 8 keep the emit kernel's LDS
// small enough for two workgroups per CU.
constexpr uint32_t kQueue = 8;

// Tokens loaded per batch by the emit loop.
constexpr uint32_t kEmitBatch = 8;

// Range encoder whose output bytes wait in a 96-bit register (p2:p1:p0,
// newest byte lowest, `nbits` = 8 x bytes held) until a carry can no longer
// reach them: a carry adds 1 to the held bytes as one integer and runs
// through any trailing 0xFF bytes by itself.  Bytes leave 4 at a time, the
// oldest first, once 10 are held, so at least 6 stay behind; a carry that
// would pass all of them (a run of 6 or more 0xFF bytes) sets the bit above
// the held bytes, which is checked whenever bytes leave.
struct RangeEncoder {
  uint32_t low, range;
  uint32_t p0, p1, p2;
  uint32_t nbits;

  // Codes the interval [cum, cum + f) of 2^15; returns the whole bytes
  // shifted out (0, 1 or 2: f >= 1 keeps range >= 2^9).
  __device__ inline uint32_t encode(uint32_t cum, uint32_t f) {
    const uint32_t r = range >> kPrec;
    // 24-bit multiplies: r < 2^17, cum and f <= 2^15
    uint32_t c;
    low = __builtin_addc(low, __umul24(r, cum), 0u, &c);
    p0 = __builtin_addc(p0, 0u, c, &c);
    p1 = __builtin_addc(p1, 0u, c, &c);
    p2 = p2 + c;
    range = __umul24(r, f);
    const uint32_t sh = lead_zeros(range) & 24u;
    append(sh);
    range <<= sh;
    return sh >> 3;
  }
  // Moves the top `sh` bits (0, 8, 16 or 24) of low into the held bytes:
  // each register takes the dword `sh` bits down in (itself : the next
  // lower one), one byte permute whose selector, bytes 7 - k .. 4 - k for
  // k = sh / 8, is the high dword of 0x0706050403020100 << sh.
  __device__ inline void append(uint32_t sh) {
    const uint32_t sel = (uint32_t)((0x0706050403020100ull << sh) >> 32);
    p2 = __builtin_amdgcn_perm(p2, p1, sel);
    p1 = __builtin_amdgcn_perm(p1, p0, sel);
    p0 = __builtin_amdgcn_perm(p0, low, sel);
    low <<= sh;
    nbits += sh;
  }
};

// Writes a stream's bytes, 4 at a time, into the payload blocks the reading
// rule gave it (queued in block order in LDS); at most `cap` bytes.
struct BlockSink {
  uint8_t *pay;      // the unit's payload
  uint32_t *queue;   // this lane's kQueue payload block numbers (LDS)
  uint32_t cnt;      // blocks of the unit handed out so far (wave-uniform)
  uint32_t head, tail;
  uint32_t slot;     // block being written (when `written` is 4 past a multiple of 8)
  uint32_t written, cap;
  bool overflow;     // more bytes than cap, or no block asked for
  bool window;       // the queue ran full, or a carry passed every held byte
  __device__ inline void push(uint32_t blk) {
    if (tail - head >= kQueue) {
      window = true;
      return;
    }
    queue[tail % kQueue] = blk;
    ++tail;
  }
  // Starts the next block: its slot is the oldest queued request.  A lane
  // with no request left (a byte count that disagrees with the statistics
  // pass, from damaged tables) stops writing for good, so every store goes
  // to a block this lane asked for, inside the unit's payload.
  __device__ inline void next_block() {
    if (head == tail) {
      overflow = true;
    } else {
      slot = queue[head % kQueue];
      ++head;
    }
  }
  // The 4 oldest held bytes of `e` (80 to 96 bits held when `take`) to the
  // stream, for the lanes with `take`.  Wave-uniform apart from `take`, and
  // written as selects: only the store itself is predicated.
  __device__ inline void take4(RangeEncoder &e, bool take) {
    const uint32_t s = (e.nbits - 64u) & 63u;  // 16..32 where taken
    // a carry past the held bytes shows as a bit at or above nbits
    const uint32_t above = (uint32_t)((uint64_t)e.p2 >> s);
    const uint32_t v = (uint32_t)((((uint64_t)e.p2 << 32) | e.p1) >> s);
    const uint32_t queued = queue[head % kQueue];
    const bool starts = take && (written & 4u) == 0;  // a new block
    const bool got = starts && head != tail;
    window = window || (take && above != 0);
    overflow = overflow || (starts && !got);
    slot = got ? queued : slot;
    head += got ? 1u : 0u;
    if (take && !overflow) put(slot * kBlock + (written & 4u), __builtin_bswap32(v));
    written += take ? 4u : 0u;
    const uint32_t kept = s >= 32u ? 0u : e.p1 & ((1u << (s & 31u)) - 1u);
    e.p1 = take ? kept : e.p1;
    e.p2 = take ? 0u : e.p2;
    e.nbits -= take ? 32u : 0u;
  }
  // A dword at byte `off` of the unit's payload, from a wave-uniform base.
  __device__ inline void put(uint32_t off, uint32_t v) {
    __asm__("" : "+v"(off));
    *reinterpret_cast<uint32_t *>(pay + off) = v;
  }
};

}  // namespace

// Statistics and exact coded length of every stream.
__global__ __launch_bounds__(kEncodeMaxWaves *kWave) void k_encode_stats(
    Desc d, const ChunkInfo *__restrict__ ci, const DecodeGroup *__restrict__ groups,
    uint32_t n_groups, uint32_t n_units, const uint8_t *__restrict__ tables,
    const uint16_t *__restrict__ kv, uint32_t T, uint8_t *__restrict__ records, int32_t *status) {
  const EncodeBlock eb = encode_block(n_groups);
  if (eb.unit >= n_units) return;
  const uint32_t ncb = (d.C + kWave - 1) / kWave;
  const uint32_t row = eb.unit / ncb, cb = eb.unit % ncb;
  const DecodeGroup gp = groups[eb.grp];
  extern __shared__ uint32_t lds_raw[];
  uint32_t *sA = lds_raw;
  uint32_t *sD = sA + kWave * kEA;
  const uint32_t lane = threadIdx.x % kWave;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const uint32_t n_waves = blockDim.x / kWave;
  const uint32_t S = n_streams(d);
  const uint32_t c0 = cb * kWave;
  const uint32_t nv = d.C - c0 < kWave ? d.C - c0 : kWave;
  const uint32_t m0 = row * d.C + c0;
  stage_tables(d, tables, m0, nv, gp.level, sA, sD);
  __syncthreads();
  if (lane >= nv) return;
  const uint32_t m = m0 + lane;
  const uint16_t *ta = reinterpret_cast<const uint16_t *>(sA + lane * kEA);
  const uint32_t third = third_of(row >> 1, d.L);
  const uint64_t ld = d.C;
  // Damaged tables are reported once, from the staged models.  The coders
  // of this pass and of emit then run the same (meaningless) range
  // evolution, so their byte counts still agree.
  if (wave == 0) {
    bool ok = model_ok(ta, 256);
    uint32_t slot = 0;
    for (uint32_t lv = 0; lv < d.nlev; ++lv) {
      if (!((gp.level >> lv) & 1u)) continue;
      const uint16_t *td = reinterpret_cast<const uint16_t *>(sD + (slot * kWave + lane) * kED);
      ok = ok && model_ok(td, (1u << d.bits[lv][third]) - 1u);
      ++slot;
    }
    if (!ok) set_status(status, KVC_ERR_CORRUPT_STREAM);
  }

  for (uint32_t i = wave; i < gp.count; i += n_waves) {
    const uint32_t k = gp.start + i;
    const ChunkInfo c = ci[k];
    const uint32_t level = c.level;
    const uint32_t lslot = __builtin_popcount(gp.level & ((1u << level) - 1u));
    const uint16_t *td = reinterpret_cast<const uint16_t *>(sD + (lslot * kWave + lane) * kED);
    const uint32_t b = d.bits[level][third];
    const int32_t M = (1 << (b - 1)) - 1;
    const uint16_t *tdM = td + M;  // entry q of it is the cumulative count of q + M
    Column x{reinterpret_cast<const uint8_t *>(kv + ((uint64_t)row * T + c.first_token) * ld + c0),
             2 * ld, 2 * lane};
    const uint32_t n = c.n_tokens;
    float lo, sa, maxabs;
    if (!stream_stats(x, n, d.G, lo, sa, maxabs)) set_status(status, KVC_ERR_NONFINITE);
    const float dl = maxabs / (float)M;
    const float inv_sa = recip_or_zero(sa), inv_dl = recip_or_zero(dl);

    // coded length = 4 + number of renormalisation shifts
    uint32_t range = 0xFFFFFFFFu;
    uint32_t shifts = 0;
    float ahat = 0.0f;
    for_each_group_token<2, kTokenBatch>(x, n, d.G, [&](float v, auto anchor) {
      uint32_t f;
      if constexpr (decltype(anchor)::value) {
        const uint32_t qa = quant_anchor(v, lo, sa, inv_sa);
        ahat = __builtin_fmaf((float)qa, sa, lo);
        f = (uint32_t)ta[qa + 1] - ta[qa];
      } else {
        const int32_t q = quant_delta(v - ahat, dl, inv_dl, M);
        f = (uint32_t)tdM[q + 1] - tdM[q];
      }
      // the encoder's update (24-bit multiply: r < 2^17, f <= 2^15)
      range = __umul24(range >> kPrec, f);
      // whole bytes to shift: 0, 1 or 2 (range >= 2^9 with f >= 1)
      const uint32_t sh = lead_zeros(range) & 24u;
      range <<= sh;
      shifts += sh >> 3;
    });
    uint32_t *rec = reinterpret_cast<uint32_t *>(records + ((uint64_t)k * S + m) * kRecBytes);
    rec[0] = __builtin_bit_cast(uint32_t, lo);
    rec[1] = __builtin_bit_cast(uint32_t, sa);
    rec[2] = __builtin_bit_cast(uint32_t, dl);
    rec[3] = 4u + shifts;
  }
}

// Container start offsets (one thread; chunk counts are small).
__global__ void k_encode_layout(Desc d, uint32_t n_chunks, const uint64_t *__restrict__ payload,
                                uint64_t *__restrict__ chunk_off_ws,
                                uint64_t *__restrict__ chunk_off_out, uint64_t out_cap,
                                uint32_t *__restrict__ fits, uint32_t *__restrict__ redo,
                                int32_t *status) {
  if (threadIdx.x != 0) return;
  redo[0] = 0;
  const uint64_t fixed = (uint64_t)kHdrBytes + (uint64_t)kRecBytes * n_streams(d);
  uint64_t acc = 0;
  for (uint32_t k = 0; k < n_chunks; ++k) {
    chunk_off_ws[k] = acc;
    chunk_off_out[k] = acc;
    acc += fixed + payload[k];
  }
  chunk_off_ws[n_chunks] = acc;
  chunk_off_out[n_chunks] = acc;
  bool ok = acc <= out_cap;
  for (uint32_t k = 0; k < n_chunks; ++k) ok = ok && payload[k] <= 0xFFFFFFFFull;
  *fits = ok ? 1u : 0u;
  if (!ok) set_status(status, KVC_ERR_CAPACITY);
}

__global__ __launch_bounds__(kEncodeMaxWaves *kWave) void k_encode_emit(
    Desc d, const ChunkInfo *__restrict__ ci, const DecodeGroup *__restrict__ groups,
    uint32_t n_groups, uint32_t n_units, const uint8_t *__restrict__ tables,
    const uint16_t *__restrict__ kv, uint32_t T, const uint8_t *__restrict__ records,
    const uint32_t *__restrict__ offsets, const uint64_t *__restrict__ chunk_off,
    const uint32_t *__restrict__ fits, uint8_t *__restrict__ out, uint32_t *__restrict__ redo,
    int32_t *status) {
  if (*fits == 0) return;
  const EncodeBlock eb = encode_block(n_groups);
  if (eb.unit >= n_units) return;
  const uint32_t ncb = (d.C + kWave - 1) / kWave;
  const uint32_t row = eb.unit / ncb, cb = eb.unit % ncb;
  const DecodeGroup gp = groups[eb.grp];
  extern __shared__ uint32_t lds_raw[];
  uint32_t *sA = lds_raw;
  uint32_t *sD = sA + kWave * kEA;
  // after the models: each lane's queue of payload block numbers
  uint32_t *queues = reinterpret_cast<uint32_t *>(sD + __builtin_popcount(gp.level) * kWave * kED);
  const uint32_t lane = threadIdx.x % kWave;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const uint32_t n_waves = blockDim.x / kWave;
  const uint32_t S = n_streams(d);
  const uint32_t c0 = cb * kWave;
  const uint32_t nv = d.C - c0 < kWave ? d.C - c0 : kWave;
  const uint32_t m0 = row * d.C + c0;
  stage_tables(d, tables, m0, nv, gp.level, sA, sD);
  __syncthreads();
  if (lane >= nv) return;
  const uint32_t m = m0 + lane;
  const uint16_t *ta = reinterpret_cast<const uint16_t *>(sA + lane * kEA);
  const uint32_t third = third_of(row >> 1, d.L);
  const uint64_t ld = d.C;

  for (uint32_t i = wave; i < gp.count; i += n_waves) {
    const uint32_t k = gp.start + i;
    const ChunkInfo c = ci[k];
    const uint32_t level = c.level;
    const uint32_t lslot = __builtin_popcount(gp.level & ((1u << level) - 1u));
    const uint16_t *td = reinterpret_cast<const uint16_t *>(sD + (lslot * kWave + lane) * kED);
    const uint32_t b = d.bits[level][third];
    const int32_t M = (1 << (b - 1)) - 1;
    const uint16_t *tdM = td + M;  // entry q of it is the cumulative count of q + M

    const uint32_t *rin =
        reinterpret_cast<const uint32_t *>(records + ((uint64_t)k * S + m) * kRecBytes);
    const float lo = __builtin_bit_cast(float, rin[0]);
    const float sa = __builtin_bit_cast(float, rin[1]);
    const float dl = __builtin_bit_cast(float, rin[2]);
    const float inv_sa = recip_or_zero(sa), inv_dl = recip_or_zero(dl);
    const uint32_t nbytes = rin[3];

    uint8_t *cont = out + chunk_off[k];
    uint32_t *rout = reinterpret_cast<uint32_t *>(cont + kHdrBytes + (uint64_t)m * kRecBytes);
    rout[0] = rin[0];
    rout[1] = rin[1];
    rout[2] = rin[2];
    rout[3] = nbytes;

    const uint32_t nblk = (uint32_t)(pad8(nbytes) / kBlock);
    BlockSink sink;
    // this unit's payload starts at its first stream's block offset
    sink.pay = cont + kHdrBytes + (uint64_t)kRecBytes * S + offsets[(uint64_t)k * S + m0];
    sink.queue = queues + (wave * kWave + lane) * kQueue;
    sink.cnt = 0;
    sink.head = sink.tail = 0;
    sink.slot = 0;
    sink.written = 0;
    sink.cap = nbytes;
    sink.overflow = false;
    sink.window = false;
    RangeEncoder enc;
    enc.low = 0;
    enc.range = 0xFFFFFFFFu;
    enc.p0 = enc.p1 = enc.p2 = 0;
    enc.nbits = 0;

    // The decoder's reading rule, run alongside: R bytes consumed by the
    // decoder, W bytes it holds, q its next block to ask for; the unit's
    // requests take consecutive payload blocks in lane order (cnt is
    // wave-uniform).  Start: blocks 0, 1, 2 of every lane.
    uint32_t cnt = 0, R = 4, W = 16, q = 0;
#pragma unroll
    for (uint32_t blk = 0; blk < 3; ++blk) {
      const bool req = blk < nblk;
      const uint64_t mask = __builtin_amdgcn_ballot_w64(req);
      if (req) {
        sink.push(cnt + lanes_below(mask));
        ++q;
      }
      cnt += (uint32_t)__builtin_popcountll(mask);
    }
    sink.cnt = cnt;

    Column x{reinterpret_cast<const uint8_t *>(kv + ((uint64_t)row * T + c.first_token) * ld + c0),
             2 * ld, 2 * lane};
    const uint32_t n = c.n_tokens;
    float ahat = 0.0f;
    uint32_t g = 0;
    for_each_token<kEmitBatch>(x, 0, 1, n, [&](float v) {
      // before this token: a reader ring with at most 8 bytes (anchor) or
      // fewer than 2 bytes (other tokens) takes its next block and asks for
      // one
      // (rare off the anchors: the whole step is skipped when no lane needs)
      const uint32_t ahead = W - R;
      const bool need = g == 0 ? ahead <= 8u : ahead < 2u;
      if (__builtin_amdgcn_ballot_w64(need) != 0) {
        const bool req = need && q < nblk;
        const uint64_t mask = __builtin_amdgcn_ballot_w64(req);
        if (req) {
          sink.push(cnt + lanes_below(mask));
          ++q;
        }
        if (need) W += kBlock;
        cnt += (uint32_t)__builtin_popcountll(mask);
        sink.cnt = cnt;
      }
      uint32_t cs, f;
      if (g == 0) {
        const uint32_t qa = quant_anchor(v, lo, sa, inv_sa);
        ahat = __builtin_fmaf((float)qa, sa, lo);
        cs = ta[qa];
        f = (uint32_t)ta[qa + 1] - cs;
      } else {
        const int32_t q = quant_delta(v - ahat, dl, inv_dl, M);
        cs = tdM[q];
        f = (uint32_t)tdM[q + 1] - cs;
      }
      g = g + 1 == d.G ? 0 : g + 1;
      // (damaged tables were reported by the statistics pass, which ran the
      // same coder on them)
      R += enc.encode(cs, f);
      const bool full = enc.nbits >= 80u;
      if (__builtin_amdgcn_ballot_w64(full) != 0) sink.take4(enc, full);
    });
    // the final 4 bytes of low, 2 at a time
#pragma unroll
    for (uint32_t h = 0; h < 2; ++h) {
      enc.append(16u);
      const bool full = enc.nbits >= 80u;
      if (__builtin_amdgcn_ballot_w64(full) != 0) sink.take4(enc, full);
    }
    // The rest (nbits <= 72): a carry past the held bytes shows as a set bit
    // at or above nbits; then zero bytes up to whole dwords, which leave the
    // oldest first, and a zero dword to complete the last block.
    {
      const uint32_t nb = enc.nbits;
      const uint64_t hi = ((uint64_t)enc.p2 << 32) | enc.p1;
      const bool lost = nb >= 32u ? (hi >> (nb - 32u)) != 0
                                  : (hi != 0 || ((uint64_t)enc.p0 >> nb) != 0);
      const uint32_t pad = (32u - (nb & 31u)) & 31u;
      enc.append(pad);  // low is spent; its bits are no longer used
      sink.window = sink.window || lost;
      uint32_t words[3] = {enc.p0, enc.p1, enc.p2};
#pragma unroll
      for (uint32_t w = 3; w-- > 0;) {
        const bool take = enc.nbits > 32u * w;
        if (take) {
          if ((sink.written & 4u) == 0) sink.next_block();
          if (sink.written + 4u > pad8(nbytes)) sink.overflow = true;
          if (!sink.overflow && !sink.window)
            sink.put(sink.slot * kBlock + (sink.written & 4u), __builtin_bswap32(words[w]));
          sink.written += 4u;
        }
      }
      if ((sink.written & 4u) != 0) {
        if (sink.written + 4u > pad8(nbytes)) sink.overflow = true;
        if (!sink.overflow && !sink.window) sink.put(sink.slot * kBlock + 4u, 0u);
        sink.written += 4u;
      }
    }
    // A lane whose queue ran full (the decoder more blocks ahead than it
    // holds) or whose carry passed every held byte has written some of its
    // bytes wrong or not at all, into blocks of this unit only; the unit is
    // coded again by k_encode_redo, which rewrites all of its blocks.
    if (!sink.window && (sink.overflow || R != nbytes || sink.written != pad8(nbytes) ||
                         q != nblk || sink.head != sink.tail))
      set_status(status, KVC_ERR_CORRUPT_STREAM);
    if (__builtin_amdgcn_ballot_w64(sink.window) != 0 && lane == 0) {
      const uint32_t e = atomicAdd(redo, 1u);
      redo[1 + 2 * e] = k;
      redo[2 + 2 * e] = eb.unit;
    }
  }
}

// The (chunk, unit)s emit listed, one workgroup (one wave) at a time, each
// lane coding one stream of the unit.  First every stream's bytes go into
// the lane's linear scratch, with a carry added into the bytes already there
// (the plain form of the coder: nothing is held back, so no run of 0xFF
// bytes is too long), and the bytes each token shifts out are recorded; then
// the reading rule is replayed over those counts, exactly as emit runs it,
// and each block asked for is copied from the scratch to its place in the
// unit's payload (a stream's padding bytes are zero).  Scratch per lane:
// pad8(4 + 2 chunk) bytes, then one byte per token.
__global__ __launch_bounds__(kWave) void k_encode_redo(
    Desc d, const ChunkInfo *__restrict__ ci, const uint8_t *__restrict__ tables,
    const uint16_t *__restrict__ kv, uint32_t T, const uint8_t *__restrict__ records,
    const uint32_t *__restrict__ offsets, const uint64_t *__restrict__ chunk_off,
    const uint32_t *__restrict__ fits, const uint32_t *__restrict__ redo,
    uint8_t *__restrict__ scratch, uint32_t lane_stride, uint8_t *__restrict__ out,
    int32_t *status) {
  if (*fits == 0) return;
  const uint32_t n_redo = redo[0];
  const uint32_t lane = threadIdx.x;
  const uint32_t ncb = (d.C + kWave - 1) / kWave;
  const uint32_t S = n_streams(d);
  const uint32_t cap = (uint32_t)pad8(4u + 2u * d.chunk);
  uint8_t *buf = scratch + ((uint64_t)blockIdx.x * kWave + lane) * lane_stride;
  uint8_t *shifts = buf + cap;
  const uint16_t *tA = reinterpret_cast<const uint16_t *>(tables + kTablesHdr);
  const uint16_t *tD =
      reinterpret_cast<const uint16_t *>(tables + kTablesHdr + (uint64_t)S * kAnchorStride * 2);
  for (uint32_t e = blockIdx.x; e < n_redo; e += gridDim.x) {
    const uint32_t k = redo[1 + 2 * e], unit = redo[2 + 2 * e];
    const uint32_t row = unit / ncb, c0 = (unit % ncb) * kWave;
    const uint32_t nv = d.C - c0 < kWave ? d.C - c0 : kWave;
    if (lane >= nv) continue;
    const uint32_t m = row * d.C + c0 + lane;
    const ChunkInfo c = ci[k];
    const uint32_t n = c.n_tokens;
    const uint32_t b = d.bits[c.level][third_of(row >> 1, d.L)];
    const int32_t M = (1 << (b - 1)) - 1;
    const uint16_t *ta = tA + (uint64_t)m * kAnchorStride;
    const uint16_t *tdM = tD + ((uint64_t)c.level * S + m) * kDeltaStride + M;
    const uint32_t *rin =
        reinterpret_cast<const uint32_t *>(records + ((uint64_t)k * S + m) * kRecBytes);
    const float lo = __builtin_bit_cast(float, rin[0]);
    const float sa = __builtin_bit_cast(float, rin[1]);
    const float dl = __builtin_bit_cast(float, rin[2]);
    const uint32_t nbytes = rin[3];
    const float inv_sa = recip_or_zero(sa), inv_dl = recip_or_zero(dl);
    const uint16_t *x = kv + ((uint64_t)row * T + c.first_token) * d.C + c0 + lane;

    // the stream's bytes, carries included
    uint64_t low = 0;
    uint32_t range = 0xFFFFFFFFu, pos = 0, g = 0;
    bool bad = false;
    float ahat = 0.0f;
    for (uint32_t j = 0; j < n; ++j) {
      const float v = h2f(x[(uint64_t)j * d.C]);
      uint32_t cs, f;
      if (g == 0) {
        const uint32_t qa = quant_anchor(v, lo, sa, inv_sa);
        ahat = __builtin_fmaf((float)qa, sa, lo);
        cs = ta[qa];
        f = (uint32_t)ta[qa + 1] - cs;
      } else {
        const int32_t q = quant_delta(v - ahat, dl, inv_dl, M);
        cs = tdM[q];
        f = (uint32_t)tdM[q + 1] - cs;
      }
      g = g + 1 == d.G ? 0 : g + 1;
      const uint32_t r = range >> kPrec;
      // (HIP's __umul24 returns int: widen the product through uint32_t)
      low += (uint64_t)(uint32_t)__umul24(r, cs);
      range = __umul24(r, f);
      if (low >> 32) {
        low &= 0xFFFFFFFFull;
        // add 1 to the bytes emitted: trailing 0xFF bytes become 0x00
        uint32_t p = pos;
        for (;;) {
          if (p == 0) {  // a carry past the first byte: impossible for valid models
            bad = true;
            break;
          }
          --p;
          const uint8_t nb = (uint8_t)(buf[p] + 1u);
          buf[p] = nb;
          if (nb != 0) break;
        }
      }
      // whole bytes out: 0, 1 or 2 (3 only for damaged tables, which the
      // statistics pass reported; it counted the same bytes)
      const uint32_t sh = lead_zeros(range) & 24u;
      for (uint32_t t = 0; t < sh; t += 8) {
        if (pos < cap) buf[pos] = (uint8_t)(low >> 24); else bad = true;
        ++pos;
        low = (low << 8) & 0xFFFFFFFFull;
      }
      range <<= sh;
      shifts[j] = (uint8_t)(sh >> 3);
    }
    for (uint32_t t = 0; t < 4; ++t) {
      if (pos < cap) buf[pos] = (uint8_t)(low >> 24); else bad = true;
      ++pos;
      low = (low << 8) & 0xFFFFFFFFull;
    }
    bad = bad || pos != nbytes;
    for (uint32_t p = pos; p < cap && (p & 7u) != 0; ++p) buf[p] = 0;

    // the reading rule, as in emit: a lane's i-th request takes the unit's
    // next payload block; requests of one step in lane order
    const uint32_t nblk = bad ? 0u : (uint32_t)(pad8(nbytes) / kBlock);
    uint8_t *pay = out + chunk_off[k] + kHdrBytes + (uint64_t)kRecBytes * S +
                   offsets[(uint64_t)k * S + row * d.C + c0];
    auto copy_block = [&](uint32_t blk, uint32_t slot) {
      const uint32_t *src = reinterpret_cast<const uint32_t *>(buf + (uint64_t)blk * kBlock);
      uint32_t *dst = reinterpret_cast<uint32_t *>(pay + (uint64_t)slot * kBlock);
      dst[0] = src[0];
      dst[1] = src[1];
    };
    uint32_t cnt = 0, R = 4, W = 16, q = 0;
    for (uint32_t blk = 0; blk < 3; ++blk) {
      const bool req = blk < nblk;
      const uint64_t mask = __builtin_amdgcn_ballot_w64(req);
      if (req) {
        copy_block(blk, cnt + lanes_below(mask));
        ++q;
      }
      cnt += (uint32_t)__builtin_popcountll(mask);
    }
    g = 0;
    for (uint32_t j = 0; j < n; ++j) {
      const uint32_t ahead = W - R;
      const bool need = g == 0 ? ahead <= 8u : ahead < 2u;
      const bool req = need && q < nblk;
      const uint64_t mask = __builtin_amdgcn_ballot_w64(req);
      if (req) {
        copy_block(q, cnt + lanes_below(mask));
        ++q;
      }
      if (need) W += kBlock;
      cnt += (uint32_t)__builtin_popcountll(mask);
      R += shifts[j];
      g = g + 1 == d.G ? 0 : g + 1;
    }
    if (bad || R != nbytes || q != nblk) set_status(status, KVC_ERR_CORRUPT_STREAM);
  }
}

__global__ void k_encode_header(Desc d, const ChunkInfo *__restrict__ ci, uint32_t n_chunks,
                                const uint8_t *__restrict__ tables,
                                const uint64_t *__restrict__ payload,
                                const uint64_t *__restrict__ chunk_off,
                                const uint32_t *__restrict__ fits, uint8_t *__restrict__ out) {
  if (*fits == 0) return;
  for (uint32_t k = threadIdx.x; k < n_chunks; k += blockDim.x) {
    const ChunkInfo c = ci[k];
    uint32_t *h = reinterpret_cast<uint32_t *>(out + chunk_off[k]);
    const uint32_t level = c.level;
    const uint64_t pid = *reinterpret_cast<const uint64_t *>(tables + 48);
    h[0] = kContainerMagic;
    h[1] = kFormatVersion | (level << 16) | (8u << 24);
    h[2] = d.G | (kPrec << 16) | ((uint32_t)d.bits[level][0] << 24);
    h[3] = (uint32_t)d.bits[level][1] | ((uint32_t)d.bits[level][2] << 8);
    h[4] = d.L;
    h[5] = d.C;
    h[6] = c.n_tokens;
    h[7] = c.first_token;
    h[8] = (uint32_t)pid;
    h[9] = (uint32_t)(pid >> 32);
    h[10] = (uint32_t)payload[k];
    h[11] = (uint32_t)(payload[k] >> 32);
    h[12] = d.chunk;
    h[13] = n_streams(d);
    h[14] = 0;
    h[15] = 0;
  }
}

// Container start offsets and the capacity check (shared with the
// refinement encoder).
hipError_t launch_encode_layout(const Desc &d, uint32_t n_chunks, const uint64_t *payload,
                                uint64_t *chunk_off_ws, uint64_t *chunk_off_out, uint64_t out_cap,
                                uint32_t *fits, uint32_t *redo, int32_t *status,
                                hipStream_t stream) {
  hipLaunchKernelGGL(k_encode_layout, dim3(1), dim3(64), 0, stream, d, n_chunks, payload,
                     chunk_off_ws, chunk_off_out, out_cap, fits, redo, status);
  return hipGetLastError();
}

hipError_t launch_index(const Desc &d, const ChunkInfo *dev_chunks, uint32_t n_chunks,
                        uint64_t *row_sums, uint32_t *flags, uint32_t *offsets, uint8_t *valid,
                        uint64_t *payload, const uint8_t *tables, int check_header_flag,
                        int32_t *status, hipStream_t stream);

size_t encode_lds_bytes(uint32_t levels) {
  return sizeof(uint32_t) * ((size_t)kWave * kEA + (size_t)levels * kWave * kED);
}

// Scratch of one k_encode_redo lane: a stream's bytes (at most 4 + 2 per
// token, in whole blocks), then one byte per token.
uint32_t encode_redo_lane_bytes(uint32_t chunk) {
  return (uint32_t)(pad8(4u + 2u * (uint64_t)chunk) + pad8(chunk));
}

// The emit kernel's LDS: the models plus every lane's block queue.
size_t encode_emit_lds_bytes(uint32_t levels, uint32_t waves) {
  return encode_lds_bytes(levels) + sizeof(uint32_t) * (size_t)waves * kWave * kQueue;
}

// Stream-ordered encode sequence; dev_chunks already holds the chunk table
// (records pointing into the workspace record array), `groups` the chunk
// groups (contiguous ranges of it) and their level masks.
hipError_t launch_encode(const Desc &d, const uint8_t *tables, const uint16_t *kv, uint32_t T,
                         const ChunkInfo *dev_chunks, uint32_t n_chunks,
                         const DecodeGroup *groups, uint32_t n_groups, uint32_t levels,
                         uint32_t waves, uint8_t *records, uint64_t *row_sums, uint32_t *flags,
                         uint32_t *offsets, uint8_t *valid, uint64_t *payload,
                         uint64_t *chunk_off_ws, uint32_t *fits, uint32_t *redo,
                         uint8_t *redo_scratch, uint32_t redo_blocks, uint8_t *out,
                         uint64_t out_cap, uint64_t *chunk_off_out, int32_t *status,
                         hipStream_t stream) {
  const uint32_t ncb = (d.C + kWave - 1) / kWave;
  const uint32_t n_units = 2u * d.L * ncb;
  const uint64_t blocks = (uint64_t)((n_units + kXcds - 1) / kXcds) * kXcds * n_groups;
  const size_t lds = encode_lds_bytes(levels);
  const size_t lds_emit = encode_emit_lds_bytes(levels, waves);
  hipLaunchKernelGGL(k_encode_stats, dim3((uint32_t)blocks), dim3(waves * kWave), lds, stream, d,
                     dev_chunks, groups, n_groups, n_units, tables, kv, T, records, status);
  hipError_t e = launch_index(d, dev_chunks, n_chunks, row_sums, flags, offsets, valid, payload,
                              tables, 0, status, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_encode_layout, dim3(1), dim3(64), 0, stream, d, n_chunks, payload,
                     chunk_off_ws, chunk_off_out, out_cap, fits, redo, status);
  hipLaunchKernelGGL(k_encode_emit, dim3((uint32_t)blocks), dim3(waves * kWave), lds_emit, stream, d,
                     dev_chunks, groups, n_groups, n_units, tables, kv, T, records, offsets,
                     chunk_off_ws, fits, out, redo, status);
  hipLaunchKernelGGL(k_encode_redo, dim3(redo_blocks), dim3(kWave), 0, stream, d, dev_chunks,
                     tables, kv, T, records, offsets, chunk_off_ws, fits, redo, redo_scratch,
                     encode_redo_lane_bytes(d.chunk), out, status);
  hipLaunchKernelGGL(k_encode_header, dim3(1), dim3(256), 0, stream, d, dev_chunks, n_chunks,
                     tables, payload, chunk_off_ws, fits, out);
  return hipGetLastError();
}

}  // namespace kvc
