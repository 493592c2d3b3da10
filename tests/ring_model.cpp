// Host-side replay of the LDS rings of the direct-to-LDS tile kernels.
//
// The kernels take every stage decision from ring_schedule.h (which stage a
// trip reads, which stages its copies write and with which K tiles, the order
// of A's and B's copies, how many copies may stay in flight at a trip's end).
// This program replays those same functions over whole K loops, in the
// kernels' loop structure -- prologue, trips, drains, the staged-C epilogue's
// scratch, the split-K flag word, the persistent grid's next-tile prologue --
// and checks the two classic hazards of a copy pipeline:
//   * a stage read before every wave's copies of its tile have landed, or
//     while another tile's copies into it may be landing;
//   * LDS that a copy, the scratch or the flag word writes while an older
//     copy into it may still land or a read of it may still be pending.
//
// Model: every wave runs the same schedule on its own share of each stage,
// and any wave may read rows that any other wave copied, so a stage is one
// unit.  Time is cut into epochs by the workgroup barriers; within an epoch
// the waves' events may interleave in any way.  A copy lands at an unknown
// time after it is issued, and is known to have landed only once a
// `vmcnt(n)` wait of its wave at the end of an epoch no longer counts it (the
// wave's last n copies may still fly).  LDS reads complete before the barrier
// that ends their epoch.
//
// Prints one line per configuration with hazards, the count of configurations
// replayed, and exits with status 1 if any hazard was found.
#include <cstdio>
#include <string>
#include <vector>

#include "ring_schedule.h"

using mihg::ring::Trip;

namespace {

struct Copy {
  int kind, stage, tile;  // kind 0 = A, 1 = B
  int issued;             // epoch
  int landed;             // epoch at whose end a wait covered it (-1: never)
  int lo, hi;             // LDS byte range of the stage
  int issue_seq;          // position in the wave's program order
  int landed_seq;         // position of the wait that covered it (-1: never)
};
struct Read {
  int kind, stage, tile, epoch, lo, hi;
};
struct Write {  // the staged-C scratch or the split-K flag word
  int epoch, lo, hi;
  const char* what;
};

struct Replay {
  std::string name;
  std::vector<Copy> copies;
  std::vector<Read> reads;
  std::vector<Write> writes;
  int epoch = 0;
  int seq = 0;  // program order of the (representative) wave
  int hazards = 0;
  int a_lo0 = 0, a_stride = 0, a_bytes = 0, b_lo0 = 0, b_stride = 0, b_bytes = 0;

  int lo_of(int kind, int stage) const {
    return kind == 0 ? a_lo0 + stage * a_stride : b_lo0 + stage * b_stride;
  }
  int bytes_of(int kind) const { return kind == 0 ? a_bytes : b_bytes; }
  void copy(int kind, int stage, int tile, int n) {
    const int lo = lo_of(kind, stage);
    for (int i = 0; i < n; ++i)
      copies.push_back(Copy{kind, stage, tile, epoch, -1, lo, lo + bytes_of(kind), seq++, -1});
  }
  void read(int kind, int stage, int tile) {
    const int lo = lo_of(kind, stage);
    reads.push_back(Read{kind, stage, tile, epoch, lo, lo + bytes_of(kind)});
    ++seq;
  }
  void write(int lo, int hi, const char* what) { writes.push_back(Write{epoch, lo, hi, what}); }
  // s_waitcnt vmcnt(n): all but this wave's last n copies have landed
  void wait(int n) {
    const int k = (int)copies.size() - n;
    for (int i = 0; i < k; ++i)
      if (copies[i].landed < 0) {
        copies[i].landed = epoch;
        copies[i].landed_seq = seq;
      }
    ++seq;
  }
  // the same for a wave that copies only operand `kind` (its vmcnt counts
  // only those copies)
  void wait_kind(int n, int kind) {
    int k = -n;
    for (const Copy& c : copies) k += c.kind == kind;
    for (Copy& c : copies) {
      if (c.kind != kind) continue;
      if (k-- <= 0) break;
      if (c.landed < 0) {
        c.landed = epoch;
        c.landed_seq = seq;
      }
    }
    ++seq;
  }
  void barrier() { ++epoch; }

  void hazard(const char* what, int a, int b) {
    if (hazards++ < 4) std::printf("  HAZARD [%s] %s (%d, %d)\n", name.c_str(), what, a, b);
  }

  void check() {
    for (const Copy& c : copies)
      if (c.landed < 0) hazard("a copy still in flight when the workgroup is done", c.kind, c.tile);
    for (const Read& r : reads) {
      int first = -1;
      for (const Copy& c : copies)
        if (c.kind == r.kind && c.stage == r.stage && c.tile == r.tile && (first < 0 || c.issued < first))
          first = c.issued;
      if (first < 0) {
        hazard("read of a tile never copied into its stage", r.kind, r.tile);
        continue;
      }
      for (const Copy& c : copies) {
        if (c.kind != r.kind || c.stage != r.stage) continue;
        if (c.tile == r.tile) {
          if (c.landed < 0 || c.landed >= r.epoch) hazard("stage read before its copies landed", r.kind, r.tile);
        } else if (c.issued >= first && c.issued <= r.epoch) {
          hazard("stage refilled while its tile is still read", r.kind, r.tile);
        }
      }
    }
    // a wave's copies go to its own rows of a stage: two copies of one wave
    // into the same LDS may not be in flight together (the older one must be
    // covered by a wait that comes before the newer one is issued)
    for (size_t i = 0; i < copies.size(); ++i)
      for (size_t j = i + 1; j < copies.size(); ++j) {
        const Copy &a = copies[i], &b = copies[j];
        if (a.hi <= b.lo || b.hi <= a.lo) continue;
        if (a.kind == b.kind && a.stage == b.stage && a.tile == b.tile) continue;
        if (a.landed_seq < 0 || a.landed_seq > b.issue_seq)
          hazard("two copies into one stage in flight", a.tile, b.tile);
      }
    // the scratch and the flag word are written and used within one epoch:
    // every copy into that LDS issued before must have landed by its start,
    // none may be issued during it, and no read of it may share the epoch
    for (const Write& w : writes) {
      for (const Copy& c : copies) {
        if (c.hi <= w.lo || w.hi <= c.lo) continue;
        if (c.issued == w.epoch || (c.issued < w.epoch && (c.landed < 0 || c.landed >= w.epoch)))
          hazard(w.what, c.kind, c.tile);
      }
      for (const Read& r : reads)
        if (!(r.hi <= w.lo || w.hi <= r.lo) && r.epoch == w.epoch) hazard(w.what, r.kind, r.tile);
    }
  }
};

// d2tile_body: BM x BN tiles, 128-byte LDS rows, SA A stages and 2 B stages,
// NW waves of WTN columns; tiles > 1: the persistent grid (one workgroup walks
// `tiles` output tiles, the next tile's first copies issued after the last
// trip of the current one).
int replay_d2(int BM, int BN, int NW, int WTN, int SA, int nk, bool sc, int tiles) {
  const int a_blk = BM / 8 / NW, b_blk = BN / 8 / NW, row = 128;
  Replay r;
  r.name = "d2tile " + std::to_string(BM) + "x" + std::to_string(BN) + " waves " + std::to_string(NW) +
           " SA " + std::to_string(SA) + " nk " + std::to_string(nk) + (sc ? " staged C" : "") +
           (tiles > 1 ? " persistent x" + std::to_string(tiles) : "");
  r.a_bytes = BM * row;
  r.b_bytes = BN * row;
  if (SA == 2) {
    const int stage = (BM + BN) * row;
    r.a_lo0 = 0, r.a_stride = stage, r.b_lo0 = BM * row, r.b_stride = stage;
  } else {
    r.a_lo0 = 0, r.a_stride = BM * row, r.b_lo0 = SA * BM * row, r.b_stride = BN * row;
  }
  const int in_flight = mihg::ring::d2_in_flight(SA, a_blk);
  // K tile ids of output tile u are u * 100000 + k, so that the tiles of
  // different output tiles never compare equal
  auto prologue = [&](int u) {
    r.copy(0, 0, u * 100000, a_blk);
    r.copy(1, 0, u * 100000, b_blk);
    for (int t = 1; t < SA - 1; ++t) r.copy(0, t, u * 100000 + t, a_blk);
  };
  prologue(0);
  for (int u = 0; u < tiles; ++u) {
    const bool more = u + 1 < tiles;
    r.wait(u == 0 ? in_flight : 0);  // later tiles: their C stores count too
    r.barrier();
    for (int kt = 0; kt < nk; ++kt) {
      const Trip t = mihg::ring::d2_trip(kt, SA);
      if (mihg::ring::d2_b_first(SA)) {
        r.copy(1, t.wb, u * 100000 + t.tb, b_blk);
        r.copy(0, t.wa, u * 100000 + t.ta, a_blk);
      } else {
        r.copy(0, t.wa, u * 100000 + t.ta, a_blk);
        r.copy(1, t.wb, u * 100000 + t.tb, b_blk);
      }
      r.read(0, t.ra, u * 100000 + kt);  // both halves read tile kt's fragments
      r.read(1, t.rb, u * 100000 + kt);
      r.wait(in_flight);
      r.barrier();
    }
    if (more) {
      r.wait(0);  // this wave's copies past the last K tile land first
      prologue(u + 1);
    }
    if (in_flight > 0 && !more) r.wait(0);
    if (sc) {
      r.barrier();
      const int scr = SA == 3 ? 2 * BM * row : 0;  // in A stage 2, else at the ring's start
      r.write(scr, scr + NW * 16 * WTN * 2, "staged-C scratch overlaps a pending copy or read");
    }
  }
  r.check();
  return r.hazards;
}

// ktile_body: BM x BN tiles, rows of 128 * KB bytes, S stages of A and SB of
// B; split: the split-K fix-up's flag word (LDS word 0); sc: staged C.
int replay_k(int BM, int BN, int NW, int WTN, int KB, int S, int SB, int nk, bool split, bool sc) {
  const int row = 128 * KB, rpb = 1024 / row;
  const int a_blk = BM / rpb / NW, b_blk = BN / rpb / NW;
  Replay r;
  r.name = "ktile " + std::to_string(BM) + "x" + std::to_string(BN) + " waves " + std::to_string(NW) +
           " K step " + std::to_string(64 * KB) + " S " + std::to_string(S) + " SB " + std::to_string(SB) +
           " nk " + std::to_string(nk) + (split ? " split-K" : "") + (sc ? " staged C" : "");
  r.a_bytes = BM * row;
  r.b_bytes = BN * row;
  if (SB == S) {
    const int stage = (BM + BN) * row;
    r.a_lo0 = 0, r.a_stride = stage, r.b_lo0 = BM * row, r.b_stride = stage;
  } else {
    r.a_lo0 = 0, r.a_stride = BM * row, r.b_lo0 = S * BM * row, r.b_stride = BN * row;
  }
  const int in_flight = mihg::ring::k_in_flight(S, SB, a_blk, b_blk);
  for (int t0 = 0; t0 < S - 1; ++t0) {
    r.copy(0, t0, t0, a_blk);
    if (t0 < SB - 1) r.copy(1, t0, t0, b_blk);
  }
  r.wait(in_flight);
  r.barrier();
  for (int kt = 0; kt < nk; ++kt) {
    const Trip t = mihg::ring::k_trip(kt, S, SB);
    if (mihg::ring::k_b_first(S, SB)) {
      r.copy(1, t.wb, t.tb, b_blk);
      r.copy(0, t.wa, t.ta, a_blk);
    } else {
      r.copy(0, t.wa, t.ta, a_blk);
      r.copy(1, t.wb, t.tb, b_blk);
    }
    r.read(0, t.ra, kt);  // every part of the trip reads tile kt's fragments
    r.read(1, t.rb, kt);
    r.wait(in_flight);
    r.barrier();
  }
  r.wait(0);
  if (split) {  // barrier, thread 0 writes the flag word, barrier
    r.barrier();
    r.write(0, 4, "split-K flag word overlaps a pending copy or read");
    r.barrier();
  }
  if (sc) {
    r.barrier();
    r.write(0, NW * 16 * WTN * 2, "staged-C scratch overlaps a pending copy or read");
  }
  r.check();
  return r.hazards;
}

// pp2tile: two groups of waves in turn, BM x BN x 64 tiles, three A stages
// and two B stages of 128-byte rows; group 1 copies A, group 0 copies B.  Each
// phase's events of both groups fall into one epoch (barrier to barrier).
int replay_pp(int BM, int BN, int WTN, int nk, bool sc) {
  const int a_blk = BM / 8 / 4, b_blk = BN / 8 / 4, row = 128;
  Replay r;
  r.name = "pp2tile " + std::to_string(BM) + "x" + std::to_string(BN) + " nk " + std::to_string(nk) +
           (sc ? " staged C" : "");
  r.a_bytes = BM * row;
  r.b_bytes = BN * row;
  r.a_lo0 = 0, r.a_stride = BM * row, r.b_lo0 = 3 * BM * row, r.b_stride = BN * row;
  const int in_a = mihg::ring::pp_in_flight_a(a_blk), in_b = mihg::ring::pp_in_flight_b(b_blk);
  // prologue
  r.copy(0, 0, 0, a_blk);  // group 1
  r.copy(0, 1, 1, a_blk);
  r.wait_kind(a_blk, 0);
  r.copy(1, 0, 0, b_blk);  // group 0
  r.wait_kind(0, 1);
  r.barrier();
  // phase -1: group 0 copies B tile 1 and reads tile 0
  r.copy(1, 1, 1, b_blk);
  r.read(0, 0, 0);
  r.read(1, 0, 0);
  r.barrier();
  for (int kt = 0; kt < nk; ++kt) {
    const Trip t = mihg::ring::pp_trip(kt);
    // phase 2kt: group 0 multiplies, then waits for B of kt+1; group 1 copies
    // A of kt+2, reads tile kt, waits
    r.wait_kind(in_b, 1);
    r.copy(0, t.wa, t.ta, a_blk);
    r.read(0, t.ra, kt);
    r.read(1, t.rb, kt);
    r.wait_kind(in_a, 0);
    r.barrier();
    // phase 2kt+1: group 1 multiplies; group 0 copies B of kt+2, reads kt+1
    r.copy(1, t.wb, t.tb, b_blk);
    if (kt + 1 < nk) {
      const Trip n = mihg::ring::pp_trip(kt + 1);
      r.read(0, n.ra, kt + 1);
      r.read(1, n.rb, kt + 1);
    }
    r.barrier();
  }
  r.wait_kind(0, 0);
  r.wait_kind(0, 1);
  if (sc) {
    r.barrier();
    r.write(2 * BM * row, 2 * BM * row + 8 * 16 * WTN * 2, "staged-C scratch overlaps a pending copy or read");
  }
  r.check();
  return r.hazards;
}

}  // namespace

int main() {
  int bad = 0, configs = 0;
  auto note = [&](int h) {
    ++configs;
    if (h) ++bad;
  };
  const int nks[] = {1, 2, 3, 4, 5, 7, 8, 31, 64, 129};
  // d2tile / d2tile3 / staged / persistent: (BM, BN, waves, wave columns)
  struct D2 { int bm, bn, nw, wtn; };
  const D2 d2s[] = {{256, 256, 8, 64}, {256, 256, 4, 128}, {256, 192, 4, 96}, {256, 128, 4, 64},
                    {128, 128, 4, 64}, {128, 64, 4, 32}, {64, 128, 4, 64}, {64, 64, 4, 32}};
  for (const D2& d : d2s)
    for (int SA : {2, 3})
      for (int nk : nks)
        for (int sc = 0; sc < 2; ++sc)
          for (int tiles : {1, 3}) {
            if (SA == 3 && (d.bm + d.bn) * 128 * 2 + d.bm * 128 > 160 * 1024) continue;
            // the persistent grid exists with three A stages only (with two, its
            // next tile's first copies would target the stage the scratch uses)
            if (tiles > 1 && SA != 3) continue;
            note(replay_d2(d.bm, d.bn, d.nw, d.wtn, SA, nk, sc, tiles));
          }
  // ktile: (BM, BN, waves, wave columns, KB, S, SB)
  struct KT { int bm, bn, nw, wtn, kb, s, sb; };
  const KT kts[] = {{128, 128, 8, 32, 2, 3, 2}, {128, 128, 4, 64, 2, 3, 2}, {128, 128, 4, 64, 2, 2, 2},
                    {128, 64, 4, 32, 2, 3, 3}, {64, 128, 4, 64, 2, 3, 3}, {64, 64, 4, 32, 2, 3, 3},
                    {64, 64, 4, 32, 4, 2, 2}, {32, 64, 4, 32, 2, 3, 3}, {32, 64, 4, 32, 4, 2, 2},
                    {16, 64, 4, 16, 4, 3, 3}, {16, 64, 4, 16, 2, 3, 3}, {16, 128, 4, 32, 2, 3, 3},
                    {16, 16, 1, 16, 4, 3, 3}, {16, 32, 2, 16, 4, 3, 3}};
  for (const KT& k : kts)
    for (int nk : nks)
      for (int split = 0; split < 2; ++split)
        for (int sc = 0; sc < 2; ++sc) note(replay_k(k.bm, k.bn, k.nw, k.wtn, k.kb, k.s, k.sb, nk, split, sc));
  // pp2tile: (BM, BN, wave columns)
  struct PP { int bm, bn, wtn; };
  const PP pps[] = {{256, 256, 64}, {256, 192, 48}, {256, 128, 32}, {128, 256, 64}};
  for (const PP& q : pps)
    for (int nk : nks)
      for (int sc = 0; sc < 2; ++sc) note(replay_pp(q.bm, q.bn, q.wtn, nk, sc));
  std::printf("replayed %d configurations, %d with hazards\n", configs, bad);
  return bad ? 1 : 0;
}
