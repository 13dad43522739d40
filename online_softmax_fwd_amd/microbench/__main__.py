import sys

from online_softmax_fwd_amd.microbench import build, run

if __name__ == "__main__":
    if "--build" in sys.argv[1:]:
        build()
    else:
        sys.exit(run())
