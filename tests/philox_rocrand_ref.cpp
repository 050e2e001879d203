// Independent Philox4x32-10 reference for the oracle's self-tests: rocRAND's
// host-callable engine.  Reads lines "seed subsequence offset" on stdin and
// prints the engine's next 32-bit output for each, in hex.
//
// rocRAND keys the generator with (seed low word, seed high word), places the
// subsequence in counter words 2-3 and offset/4 in counter words 0-1, and
// returns output word (offset mod 4) of that counter.  So word j of Philox at
// counter (a, b, c, d) is engine(seed, c + d*2^32, 4*(a + b*2^32) + j).next().
#include <cstdio>
#include <rocrand/rocrand_philox4x32_10.h>

int main() {
  unsigned long long seed, subseq, offset;
  while (std::scanf("%llu %llu %llu", &seed, &subseq, &offset) == 3) {
    rocrand_device::philox4x32_10_engine eng(seed, subseq, offset);
    std::printf("%08x\n", eng.next());
  }
  return 0;
}
