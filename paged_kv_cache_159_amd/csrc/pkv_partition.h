// Body of the decode partition kernel, shared by the plain decode launch and
// the grouped decode launch (whose tail partitions run the same code).
#pragma once

#include "pkv_device.h"

namespace pkv {

constexpr int kWaves = 8;
typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
// 16-token tiles each loop step covers: every wave has 2 * (tiles per step)
// rows of K and V in flight per step. The plain decode takes one (two
// measured within +-0.5 points at the LLaMA-7B and long-context decodes);
// the grouped call's tail partitions take two: they share the machine with
// the shared-prefix units, and the longest tails bound the launch, so more
// bytes in flight per tail workgroup shortened the shared-prefix decode
// (grouped call 69.9-70.0 -> 69.2-69.4 us on two boxes; block size 8
// 69.3-70.0 -> 68.2-68.6, block size 32 70.1-70.4 -> 68.6-69.5).
constexpr int kTilesPerStep = 1;
constexpr int kTailTilesPerStep = 2;

// LDS bytes partition_body needs: per wave and head (max, sum), and per wave a
// head group's accumulators.
template <int D>
constexpr int partition_lds_bytes() {
  constexpr int HG = 64 / (D / 8);
  return (2 * kWaves * HG + kWaves * HG * D) * (int)sizeof(float);
}

// Work-item order of the plain decode grid. The grid holds num_parts
// partition slots per sequence (sized from the table), of which a sequence
// uses ceil(ctx / PT). A full partition (PT tokens) is the longest item; each
// sequence has at most one shorter item, its last partition. The real items
// are dispatched longest first: every full partition (sequence-major), then
// the last partitions by length class (kRemClasses classes of PT /
// kRemClasses tokens, longest class first, sequences in order within a
// class), so the items still running when the grid drains are the shortest
// ones. Measured on MI355X against partition-major order (32 heads x 128,
// fp16): 64 sequences of U[128, 2048] tokens 169.7 -> 164.3 us, 64 of
// Exp(512) 87.5 -> 83.5, 128 of U[128, 2048] 372.0 -> 361.5, 256 of
// U[128, 2048] 690.4 -> 682.5, 256 of Exp(512) and 8 x 32K unchanged
// (351.7, 633.7 -> 629.0). The plan is not free: per-workgroup timestamps put
// ~1.3 us between a workgroup's start and its first item load (the context
// lengths' load, then a dependent chain of ~150 instructions issued by all
// 8 waves), which loses where items are short, e.g. 8 beams per prompt
// reading shared blocks (97 -> 108 us); there the longest-first order has
// little to balance.
constexpr int kPlanMaxSeqs = 256;   // context lengths held in registers (4 per lane)
constexpr int kRemClasses = 8;

// Backed-up items. The XCDs of one MI355X run the same work at different
// speeds (per-workgroup timestamps: up to ~10% apart, which XCDs are slow
// varies by box), and the hardware hands every XCD the same share of the
// grid. So the last quarter of the item order (at most backup_capacity items)
// also gets a second, backup workgroup, appended to the grid on the next XCD:
// whichever of the two claims the item first computes it, the other exits.
// An XCD that has run through its own share takes over a slower XCD's last
// items. The host gives claim flags (and so backups) only to planned orders
// over 512-token partitions, whose items are long. Measured on MI355X
// (decode call, HIP-event medians, interleaved runs): 8 x 32K tokens
// 634-638 -> 625-627 us on five runs (the XCDs' end times 570-629 -> 602-621
// us), 256 of Exp(512) 340-342 -> 338-340 us. Over 256-token partitions the
// backups gained nothing at 64 of U[128, 2048] and cost beam search through
// the plain call 4% (short items over shared blocks pay the claim for
// little); backing up half the order instead of a quarter cost 2-3%.
__host__ __device__ inline int backup_capacity(int num_seqs, int num_parts) {
  return (num_seqs * num_parts + 3) / 4;
}

// Item of grid slot sp (of num_seqs * num_parts slots), or with bk >= 0 the
// item of backup workgroup bk (the bk-th item of the backed-up range, the
// last B of the N items, B = min(backup_items, ceil(N / 4))): sequence s,
// partition p and the sequence's context length ctx (read from the registers
// the plan already holds); false for a slot or backup with no item. claim_k
// is the item's index in the backed-up range, -1 outside it. Computed by each
// wave from the context lengths (one load per lane and 64 sequences),
// wave-uniform.
template <int PT, bool BACKUP>
__device__ __forceinline__ bool plan_item(int sp, int bk, int backup_items, int num_seqs,
                                          int num_parts,
                                          const int32_t* __restrict__ context_lens, int& s,
                                          int& p, int& ctx, int& claim_k) {
  constexpr int KC = kPlanMaxSeqs / 64;
  const int lane = threadIdx.x & 63;
  int cl[KC];
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    const int sq = 64 * k + lane;
    cl[k] = (64 * k < num_seqs && sq < num_seqs) ? context_lens[sq] : 0;
  }
  int nf[KC], cls[KC], incl[KC], tot[KC];
  int F = 0, R = 0;
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    nf[k] = (int)((uint32_t)cl[k] / PT);
    const int r = (int)((uint32_t)cl[k] % PT);
    cls[k] = r ? (r * kRemClasses + PT - 1) / PT : 0;   // 1 .. kRemClasses
    incl[k] = 0;
    tot[k] = 0;
    if (64 * k < num_seqs) {                             // wave-uniform
      incl[k] = wave_inclusive_scan(nf[k]);
      tot[k] = __builtin_amdgcn_readlane(incl[k], 63);
      F += tot[k];
      R += __popcll(__ballot(r > 0));
    }
  }
  const uint32_t N = (uint32_t)(F + R);                  // real items
  // Item i sits at slot floor(i * NP / N): the empty slots are spread evenly
  // over the grid. Gathered at the grid's end instead, they cost 10% at 256
  // sequences (~11,000 empty workgroups, each loading the context lengths,
  // run after the real work has drained).
  const uint32_t NP = (uint32_t)num_seqs * (uint32_t)num_parts;
  uint32_t i;
  if constexpr (BACKUP) {
    const uint32_t B = min((uint32_t)backup_items, (N + 3) / 4);   // backed-up items: [N - B, N)
    if (bk < 0) {
      i = ((uint32_t)sp * N + NP - 1) / NP;
      if (i >= N || (i * NP) / N != (uint32_t)sp) return false;
    } else {
      if ((uint32_t)bk >= B) return false;
      i = N - B + (uint32_t)bk;
    }
    claim_k = i >= N - B ? (int)(i - (N - B)) : -1;
  } else {
    i = ((uint32_t)sp * N + NP - 1) / NP;
    if (i >= N || (i * NP) / N != (uint32_t)sp) return false;
  }
  if ((int)i < F) {
    int j = (int)i;
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      if (j < tot[k]) {
        const int ln = __ffsll((unsigned long long)__ballot(incl[k] > j)) - 1;
        s = 64 * k + ln;
        p = j - __builtin_amdgcn_readlane(incl[k] - nf[k], ln);
        ctx = __builtin_amdgcn_readlane(cl[k], ln);
        return true;
      }
      j -= tot[k];
    }
    return false;   // not reached: i < F
  }
  int j = (int)i - F;
#pragma unroll
  for (int c = kRemClasses; c >= 1; --c) {
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      if (64 * k >= num_seqs) break;
      const uint64_t m = __ballot(cls[k] == c);
      const int cnt = __popcll(m);
      if (j < cnt) {
        const int ln = nth_set_lane(m, j);
        s = 64 * k + ln;
        p = __builtin_amdgcn_readlane(nf[k], ln);
        ctx = __builtin_amdgcn_readlane(cl[k], ln);
        return true;
      }
      j -= cnt;
    }
  }
  return false;     // not reached: i < N
}

// Sequence of the grouped call's first-tail-partition slot sp (of num_seqs
// slots): sequences by context length, longest first (kTailClasses classes
// over the batch's range of lengths, sequences in order within a class), so
// the tails that run last are the short ones. The tail is the context past
// the group's shared prefix; ordering by the whole context is exact when
// the groups share prefixes of one length and close otherwise. Returns -1
// when the batch is too large to rank (the caller keeps slot order).
constexpr int kTailClasses = 16;
__device__ __forceinline__ int plan_tail_seq(int sp, int num_seqs,
                                             const int32_t* __restrict__ context_lens) {
  constexpr int KC = kPlanMaxSeqs / 64;
  if (num_seqs > kPlanMaxSeqs) return -1;
  const int lane = threadIdx.x & 63;
  int cl[KC];
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    const int sq = 64 * k + lane;
    cl[k] = (64 * k < num_seqs && sq < num_seqs) ? context_lens[sq] : -1;
  }
  int mx = INT_MIN, mn = INT_MAX;
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    if (64 * k < num_seqs) {   // wave-uniform
      mx = max(mx, wave_max(cl[k]));
      mn = min(mn, -wave_max(cl[k] < 0 ? INT_MIN + 1 : -cl[k]));
    }
  }
  const int span = mx - mn + 1;
  int cls[KC];
#pragma unroll
  for (int k = 0; k < KC; ++k)
    cls[k] = cl[k] < 0 ? -1 : (int)(((int64_t)(mx - cl[k]) * kTailClasses) / span);
  int j = sp;
#pragma unroll 1
  for (int c = 0; c < kTailClasses; ++c) {
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      if (64 * k >= num_seqs) break;
      const uint64_t m = __ballot(cls[k] == c);
      const int cnt = __popcll(m);
      if (j < cnt) return 64 * k + nth_set_lane(m, j);
      j -= cnt;
    }
  }
  return -1;   // not reached: sp < num_seqs
}

// Grid slots of the plain launch whose items plan_item orders (above this the
// grid keeps its plain order, partition-major): slot arithmetic stays in 32
// bits.
__host__ __device__ constexpr bool plan_fits(int num_seqs, int num_parts) {
  return num_parts > 1 && num_seqs <= kPlanMaxSeqs && (int64_t)num_seqs * num_parts <= 65536;
}

// One workgroup (index wg) of the partition launch: (head group, sequence,
// partition), head groups fastest, over blocks of BS tokens. The partition is
// walked in 16-token tiles whatever the block size (a tile is one 16-token
// block, half a 32-token block or two 8-token blocks): wave w reads tokens w
// and w + 8 of every tile, each through the block table. TAIL = true is the
// grouped call's tail:
// each sequence starts after its group's shared-prefix tiles (handled by the
// shared-prefix units), its partitions go to partial slots slot_base + p,
// every partition writes a partial (the merge always runs), and the sequence's
// shared-prefix token count goes to seq_tok0[s] for the merge.
template <typename T, int D, int PT, int BS, bool TAIL, bool BACKUP = false>
__device__ __forceinline__ void partition_body(
    int wg, uint16_t* __restrict__ out, float* __restrict__ ws_ml, float* __restrict__ ws_o,
    const uint16_t* __restrict__ query, const uint16_t* __restrict__ key_cache,
    const uint16_t* __restrict__ value_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, int num_seqs, int num_heads, int max_blocks,
    int num_parts, float scale_log2, const int32_t* __restrict__ group_start,
    const int32_t* __restrict__ shared_blocks, int num_groups, int slot_base,
    int32_t* __restrict__ seq_tok0, uint8_t* lds, uint32_t* __restrict__ flags = nullptr,
    int backup_items = 0) {
  using E = Elem<T>;
  constexpr int LPR = D / 8;         // lanes per head row (16 bytes each)
  constexpr int HG = 64 / LPR;       // heads per wave-wide load
  constexpr int TPS = TAIL ? kTailTilesPerStep : kTilesPerStep;
  constexpr int STEP = kTileTokens * TPS;             // tokens per loop step
  constexpr int RPW = STEP / kWaves;                  // rows each wave reads per step
  static_assert(PT % BS == 0 && PT % STEP == 0, "partition is whole blocks and steps");
  static_assert(BS % 8 == 0, "rows w, w + 8, ... of a step lie in blocks of >= 8 tokens");
  static_assert(PT / BS <= 64, "a partition's table entries fit one per lane");

  const int H = num_heads;
  const int groups = (H + HG - 1) / HG;
  // BACKUP: workgroups past the grid's num_seqs * num_parts slots are
  // backups: backup bk takes the head group one below its position's, so it
  // runs on the XCD after the one its item's first workgroup runs on (the
  // hardware deals workgroup ids to the 8 XCDs in turn, and the slots hold
  // whole multiples of 8 workgroups at head size 128).
  static_assert(!(TAIL && BACKUP), "backups are for the planned plain order");
  const int prim_wgs = num_seqs * num_parts * groups;
  const bool is_backup = BACKUP && wg >= prim_wgs;
  const int g = is_backup ? ((wg - prim_wgs) % groups + groups - 1) % groups : wg % groups;
  const int sp = is_backup ? 0 : wg / groups;
  const int bk = is_backup ? (wg - prim_wgs) / groups : -1;
  int claim_k = -1;
  int s = sp % num_seqs;
  int p = sp / num_seqs;
  if constexpr (TAIL) {
    if (p == 0) {   // first tail partitions: longest contexts first
      const int ts = plan_tail_seq(s, num_seqs, context_lens);
      if (ts >= 0 && ts < num_seqs) s = __builtin_amdgcn_readfirstlane(ts);
    }
  }
  int planned_ctx = -1;   // the item's context length when the plan gave it
  if constexpr (!TAIL) {
    if (plan_fits(num_seqs, num_parts)) {
      int ps = 0, pp = 0, pc = 0;
      const bool real = plan_item<PT, BACKUP>(sp, bk, backup_items, num_seqs, num_parts,
                                              context_lens, ps, pp, pc, claim_k);
      // an item outside the grid's (sequence, partition) range is never
      // produced; the bound keeps every later index inside the arrays anyway
      if (!real || (unsigned)ps >= (unsigned)num_seqs || (unsigned)pp >= (unsigned)num_parts)
        return;
      s = __builtin_amdgcn_readfirstlane(ps);
      p = __builtin_amdgcn_readfirstlane(pp);
      planned_ctx = __builtin_amdgcn_readfirstlane(pc);
    }
  }
  if constexpr (TAIL) {
    // A later tail partition starts at least p * PT tokens in: past the
    // context it has nothing to do, known from the context length alone
    // (most of these slots are empty: tails are usually shorter than PT).
    if (p > 0 && p * PT >= context_lens[s]) return;
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int hl = lane / LPR;          // head within the group
  const int c = lane % LPR;           // 8-element column chunk
  const int h = g * HG + hl;
  const bool head_ok = h < H;
  const int hr = head_ok ? h : 0;     // lanes past the last head read head 0 and are ignored

  // Loads that depend only on (s, p, g) go out first, together: the query,
  // the context length (unless the item plan already holds it), the
  // partition's table entries (plain partitions) or the first 64 entries and
  // the group lookup (tails). A tail's first block is known only after the
  // group lookup, so its entries are read from this speculative copy when
  // they lie in it. Either way the table load does not wait for another
  // memory round trip.
  const uint4 qv = *reinterpret_cast<const uint4*>(query + ((size_t)s * H + hr) * D + c * 8);
  int32_t table_spec = 0;
  if constexpr (TAIL) {
    table_spec = lane < max_blocks ? block_tables[(size_t)s * max_blocks + lane] : 0;
  } else {
    // The partition's PT / BS entries (those inside the table): a superset of
    // the ones its tokens use, loaded without waiting for the context length.
    const int e = p * (PT / BS) + lane;
    table_spec = (lane < PT / BS && e < max_blocks) ? block_tables[(size_t)s * max_blocks + e] : 0;
  }
  if (BACKUP && claim_k >= 0) {
    // A backed-up item: its flag is claimed exactly twice per launch (first
    // and backup workgroup) with a wrapping increment that counts 0 -> 1 -> 0,
    // and the claim that finds 0 computes the item. From a zeroed flag the
    // first arrival wins and the flag ends at zero again; from any other
    // value the second claim finds 0, so exactly one workgroup computes the
    // item whatever the workspace held. Issued after the query and table
    // loads, which fly meanwhile.
    __shared__ uint32_t s_won;
    if (threadIdx.x == 0) {
      const uint32_t old = __builtin_amdgcn_atomic_inc32(
          flags + (size_t)claim_k * groups + g, 1u, __ATOMIC_RELAXED, "agent");
      s_won = old == 0u;
    }
    __syncthreads();
    if (!s_won) return;
  }
  const int ctx = planned_ctx >= 0 ? planned_ctx : context_lens[s];
  int tok0 = 0;   // first token this launch covers for sequence s
  if constexpr (TAIL)
    tok0 = shared_prefix_tokens(group_shared_blocks(s, group_start, shared_blocks, num_groups), BS);
  if constexpr (TAIL) {
    if (p == 0 && g == 0 && threadIdx.x == 0) seq_tok0[s] = tok0;
  }
  const int tok_begin = tok0 + p * PT;
  if (tok_begin >= ctx) return;
  const int tok_end = min(ctx, tok_begin + PT);
  // tok0 (a multiple of 16) and PT are multiples of the tile and the block
  const int nsteps = (tok_end - tok_begin + STEP - 1) / STEP;

  // The partition's table entries, one per lane (at most 64), loaded once;
  // the loop reads them with v_readlane (no memory latency per step): entry
  // j sits in lane j - tbase of table_lane.
  const uint32_t blk0 = (uint32_t)tok_begin / BS;
  const int nblk = (tok_end - tok_begin + BS - 1) / BS;
  int32_t table_lane;
  uint32_t tbase = blk0;              // table entry held by lane 0
  if constexpr (!TAIL) {
    table_lane = table_spec;       // entry blk0 + j in lane j
  } else if (blk0 + nblk <= 64) {
    table_lane = table_spec;
    tbase = 0;
  } else {
    table_lane = lane < nblk ? block_tables[(size_t)s * max_blocks + blk0 + lane] : 0;
  }
  const uint32_t kv_dim = (uint32_t)H * D;
  const size_t blk_bytes = (size_t)BS * kv_dim * sizeof(uint16_t);
  const uint32_t row_bytes = kv_dim * (uint32_t)sizeof(uint16_t);
  const uint32_t col_bytes = ((uint32_t)hr * D + (uint32_t)c * 8) * sizeof(uint16_t);
  const char* kpool = reinterpret_cast<const char*>(key_cache);
  const char* vpool = reinterpret_cast<const char*>(value_cache);

  float m = -INFINITY, l = 0.f;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;

  for (int k = 0; k < nsteps; ++k) {
    const int tb = tok_begin + k * STEP;   // < ctx
    // Token tb + wave + 8i, wave-uniform. Tokens past the context re-read the
    // step's first token (valid, a cache hit) instead of branching; their
    // weight is exactly 0 below. Address: the block's base (64-bit, scalar)
    // plus the row and the lane's column (32-bit).
    uint4 kr[RPW], vr[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const uint32_t t = (uint32_t)(tb + wave + i * kWaves);
      const uint32_t te = t < (uint32_t)ctx ? t : (uint32_t)tb;
      // With one tile per step at block sizes >= 16, the tile sits in the
      // block of tb.
      const uint32_t bi =
          ((TPS == 1 && BS >= kTileTokens) ? (uint32_t)tb : te) / BS - tbase;
      const uint32_t phys = (uint32_t)__builtin_amdgcn_readlane(table_lane, bi);
      const uint32_t off = (te % BS) * row_bytes + col_bytes;
      // Non-temporal V loads: a row read once per launch should not displace
      // other lines (+5-7% at the LLaMA-7B and long-context decodes). K stays
      // cached in the plain call, whose blocks may be shared by several
      // sequences (beam search through this call keeps more of its cache
      // hits); tail partitions read private blocks and load both
      // non-temporally.
      const char* kp = kpool + (size_t)phys * blk_bytes + off;
      if constexpr (TAIL)
        kr[i] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(kp)));
      else
        kr[i] = *reinterpret_cast<const uint4*>(kp);
      vr[i] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(
                                            reinterpret_cast<const u32x4_nt*>(vpool + (size_t)phys * blk_bytes + off)));
    }
    float sc[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      float d = E::dot2(kr[i].x, qv.x, 0.f);
      d = E::dot2(kr[i].y, qv.y, d);
      d = E::dot2(kr[i].z, qv.z, d);
      d = E::dot2(kr[i].w, qv.w, d);
      d = group_sum<LPR>(d);
      sc[i] = (tb + wave + i * kWaves < ctx) ? d * scale_log2 : -INFINITY;
    }
    float bm = sc[0];
#pragma unroll
    for (int i = 1; i < RPW; ++i) bm = fmaxf(bm, sc[i]);
    const float mn = fmaxf(m, bm);
    // While a stream has seen no valid row, m and mn are -inf; using 0 as the
    // reference then makes every weight 2^-inf = 0 without a branch (a
    // divergent branch here would make the compiler wait for all loads).
    const float ref = (mn == -INFINITY) ? 0.f : mn;
    const float alpha = fast_exp2(m - ref);
    l *= alpha;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= alpha;
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const float pw = fast_exp2(sc[i] - ref);
      l += pw;
      acc[0] += pw * E::lo(vr[i].x);
      acc[1] += pw * E::hi(vr[i].x);
      acc[2] += pw * E::lo(vr[i].y);
      acc[3] += pw * E::hi(vr[i].y);
      acc[4] += pw * E::lo(vr[i].z);
      acc[5] += pw * E::hi(vr[i].z);
      acc[6] += pw * E::lo(vr[i].w);
      acc[7] += pw * E::hi(vr[i].w);
    }
    m = mn;
  }

  // Merge the waves' streams of each head through LDS.
  float(*s_m)[HG] = reinterpret_cast<float(*)[HG]>(lds);
  float(*s_l)[HG] = reinterpret_cast<float(*)[HG]>(lds + kWaves * HG * sizeof(float));
  float(*s_acc)[HG * D] =
      reinterpret_cast<float(*)[HG * D]>(lds + 2 * kWaves * HG * sizeof(float));
#pragma unroll
  for (int j = 0; j < 8; ++j) s_acc[wave][hl * D + c * 8 + j] = acc[j];
  if (c == 0) {
    s_m[wave][hl] = m;
    s_l[wave][hl] = l;
  }
  __syncthreads();
  const int parts_s = TAIL ? 0 : (ctx + PT - 1) / PT;
  for (int o = threadIdx.x; o < HG * D; o += kWaves * 64) {
    const int ol = o / D;
    const int d = o % D;
    const int oh = g * HG + ol;
    if (oh >= H) break;   // o grows, so later o are past H too
    float M = s_m[0][ol];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][ol]);
    float L = 0.f, val = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float cw = (s_m[w][ol] == -INFINITY) ? 0.f : fast_exp2(s_m[w][ol] - M);
      L += s_l[w][ol] * cw;
      val += s_acc[w][o] * cw;
    }
    if (parts_s == 1) {
      out[((size_t)s * H + oh) * D + d] = E::round(val / L);
    } else {
      const size_t pi = ((size_t)s * H + oh) * num_parts + slot_base + p;
      ws_o[pi * D + d] = val / L;
      if (d == 0) {
        ws_ml[pi * 2] = M;
        ws_ml[pi * 2 + 1] = L;
      }
    }
  }
}

}  // namespace pkv
