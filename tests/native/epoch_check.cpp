// Host-side check of the epoch bookkeeping of the fused launches (epochs.hpp):
// the epoch handed to a launch is the family's count of enqueued launches plus
// one; a launch that fails to enqueue does not move the count (else every later
// eager exchange would wait for an epoch the device never completes); a
// captured launch switches the plan to epochs inferred on the device (0) for
// good; reset clears the counts. Built and run by tests/test_host_sanitizers.py.
#include <cstdio>

#include "epochs.hpp"

namespace {

int fails = 0;

void expect(bool ok, const char *what)
{
    if (!ok) {
        std::printf("FAIL: %s\n", what);
        ++fails;
    }
}

}  // namespace

int main()
{
    halo::EpochBook<3> b;
    expect(b.next(0, false) == 1u, "first launch gets epoch 1");
    b.launched(0, true);
    expect(b.next(0, false) == 2u, "second launch gets epoch 2");
    b.launched(0, false);  // failed to enqueue
    expect(b.next(0, false) == 2u, "a failed launch leaves the count");
    b.launched(0, true);
    expect(b.next(0, false) == 3u, "the count moves on after a success");
    expect(b.next(1, false) == 1u, "families count apart");
    b.launched(1, true);
    b.launched(1, true);
    expect(b.next(1, false) == 3u, "family 1 counted twice");
    expect(b.next(0, false) == 3u, "family 0 unchanged by family 1");
    // wrap: a count of 2^32 - 1 hands out 0 once (inferred on the device)
    b.count[2] = 0xffffffffu;
    expect(b.next(2, false) == 0u, "wrap asks for inference");
    b.launched(2, true);
    expect(b.next(2, false) == 1u, "after the wrap the count restarts");
    b.reset();
    expect(b.next(0, false) == 1u && b.next(1, false) == 1u, "reset clears the counts");
    // capture: 0 from then on, the eager counts stop
    expect(b.next(0, true) == 0u, "a captured launch infers its epoch");
    b.launched(0, true);
    expect(b.on_device, "capture switches to inferred epochs");
    expect(b.next(0, false) == 0u && b.next(1, false) == 0u, "every later launch infers");
    std::printf("%d epoch check(s) failed\n", fails);
    return fails ? 1 : 0;
}
