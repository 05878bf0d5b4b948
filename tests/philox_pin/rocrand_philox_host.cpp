// Test helper: rocRAND's Philox4x32-10 engine, compiled host-side, used as an
// independent library implementation of the generator to pin the oracle's
// Philox against. It is never linked into the HIP library or the oracle.
#include <rocrand/rocrand_philox4x32_10.h>

extern "C" void pin_philox4x32_10(unsigned long long seed, const unsigned int *ctr,
                                  unsigned int *out)
{
    // rocRAND places `subsequence` in counter words 2..3 and offset/4 in
    // words 0..1, so this reproduces the block at counter (c0, c1, c2, c3).
    unsigned long long subsequence = ((unsigned long long)ctr[3] << 32) | ctr[2];
    unsigned long long block = ((unsigned long long)ctr[1] << 32) | ctr[0];
    rocrand_device::philox4x32_10_engine engine(seed, subsequence, 0);
    engine.discard(block);
    engine.discard(block);
    engine.discard(block);
    engine.discard(block);
    uint4 r = engine.next4();
    out[0] = r.x;
    out[1] = r.y;
    out[2] = r.z;
    out[3] = r.w;
}
