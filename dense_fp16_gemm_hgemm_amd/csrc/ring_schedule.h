// Stage arithmetic of the LDS rings of the direct-to-LDS tile kernels:
// which stage a trip reads, which stages its copies write, which K tiles
// those copies carry, the order they are issued in, and how many copies a
// wave may leave in flight at a trip's end.  The kernels take every one of
// these decisions from here, and a host-side model (tests/test_ring_hazards.py)
// replays the same functions over whole K loops to check that no stage is
// read before its copies have landed or overwritten while it may still be
// read.  [P3] "B-08. Hopper TMA：从单线程 Bulk Copy 到吞吐墙" (lqnn.cn) §3.3-§3.4
// lists exactly those two mistakes (reading a stage before it has landed,
// refilling it while it is in use) as the classic ones of a copy pipeline.
//
// Plain constexpr integer functions: they compile for the host and the device.
#pragma once

namespace mihg {
namespace ring {

#if defined(__HIPCC__)
#define MIHG_RING_FN __host__ __device__ constexpr inline
#else
#define MIHG_RING_FN constexpr inline
#endif

// One trip kt of a K loop: tile kt is read from A stage ra and B stage rb;
// the trip's copies bring A tile ta into A stage wa and B tile tb into B
// stage wb.
struct Trip {
  int ra, rb;
  int wa, wb;
  int ta, tb;
};

// d2tile family: SA = 2 or 3 stages of A, 2 of B.  A is copied SA - 1 tiles
// ahead, B one tile ahead; a copy refills the stage that tile kt - 1 used.
MIHG_RING_FN Trip d2_trip(int kt, int SA) {
  const int ra = SA == 2 ? (kt & 1) : kt % 3;
  const int rb = kt & 1;
  Trip t{};
  t.ra = ra;
  t.rb = rb;
  t.wa = SA == 2 ? (ra ^ 1) : (ra == 0 ? 2 : ra - 1);
  t.wb = rb ^ 1;
  t.ta = kt + SA - 1;
  t.tb = kt + 1;
  return t;
}
// d2tile: within a trip, are B's copies issued before A's?  With three A
// stages they are, so the trip-end wait can leave exactly A's in flight.
MIHG_RING_FN bool d2_b_first(int SA) { return SA == 3; }
// d2tile: copies a wave may leave in flight at a trip's end (and after the
// prologue), a_blk being its A copies per trip: the A copies of the tile two
// ahead with three A stages, none with two.
MIHG_RING_FN int d2_in_flight(int SA, int a_blk) { return SA == 3 ? a_blk : 0; }

// ktile family: S stages of A and SB (= S or S - 1) of B.  A is copied S - 1
// tiles ahead, B SB - 1 tiles ahead.
MIHG_RING_FN Trip k_trip(int kt, int S, int SB) {
  Trip t{};
  t.ra = kt % S;
  t.rb = SB == S ? t.ra : kt % SB;
  t.wa = (kt + S - 1) % S;
  t.wb = SB == S ? t.wa : (kt + SB - 1) % SB;
  t.ta = kt + S - 1;
  t.tb = kt + SB - 1;
  return t;
}
// ktile: B's copies first when B has one stage fewer (its copies must land a
// trip earlier than A's).
MIHG_RING_FN bool k_b_first(int S, int SB) { return SB != S; }
MIHG_RING_FN int k_in_flight(int S, int SB, int a_blk, int b_blk) {
  return a_blk * (S - 2) + b_blk * (SB - 2);
}

// pp2tile (two groups of waves taking turns at the matrix pipes, one full K
// tile per turn): 3 stages of A, 2 of B, both copied two tiles ahead.  K tile
// kt is read by group 0 in phase 2kt-1 and by group 1 in phase 2kt; group 1
// copies A tile kt+2 in phase 2kt (into the stage tile kt-1 left), group 0
// copies B tile kt+2 in phase 2kt+1 (into the stage tile kt leaves).
MIHG_RING_FN Trip pp_trip(int kt) {
  Trip t{};
  t.ra = kt % 3;
  t.rb = kt & 1;
  t.wa = (kt + 2) % 3;
  t.wb = kt & 1;
  t.ta = kt + 2;
  t.tb = kt + 2;
  return t;
}
// pp2tile: copies a group's wave may leave in flight when its turn at the
// matrix pipes or at memory ends: group 1 (A) the tile it just issued, group 0
// (B) none, at the end of its compute phase (the tile issued a phase before).
MIHG_RING_FN int pp_in_flight_a(int a_blk) { return a_blk; }
MIHG_RING_FN int pp_in_flight_b(int) { return 0; }

#undef MIHG_RING_FN

}  // namespace ring
}  // namespace mihg
