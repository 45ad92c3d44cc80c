#!/bin/sh
# Builds the fp64 CPU oracle (test infrastructure) next to this script.
#   build.sh                  liboracle_conv3x3.so, gcc
#   build.sh --sanitize OUT   OUT, clang with AddressSanitizer and
#                             UndefinedBehaviorSanitizer (the CPU tests' sanitizer run;
#                             the process needs clang's sanitizer runtime preloaded)
set -e
cd "$(dirname "$0")"
if [ "$1" = "--sanitize" ]; then
  /opt/rocm/lib/llvm/bin/clang -O1 -g -fopenmp -fPIC -shared -Wall -Wextra -std=c11 \
    -fsanitize=address,undefined -fno-sanitize-recover=all -fno-omit-frame-pointer \
    -o "$2" conv3x3_oracle.c -lm
else
  gcc -O2 -fopenmp -fPIC -shared -Wall -Wextra -std=c11 -o liboracle_conv3x3.so conv3x3_oracle.c -lm
fi
